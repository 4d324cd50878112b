// route.hip -- router logits (fp64 accumulation) fused with softmax top-k and
// renormalised weights.
//
// Router: a small linear layer gives every expert a score for the token,
// followed by softmax and top-k (Baidu "MoE稀疏架构是什么" page, section 三.1
// and the section 四 pseudocode; qqiyuan MoE guide, MoELayer pseudocode).
// The selected probabilities are renormalised over the k picked experts
// (Baidu page, section 四: softmax over the top-k scores); softmax over all
// experts followed by renormalisation is the same quantity, so the kernel
// evaluates w_j = exp(l_j - l_max) / sum_{i<k} exp(l_i - l_max) directly.
// Ranking: larger fp64 logit first, equal logits to the lower expert index.
//
// Products of bf16 (or fp32) inputs are exact in fp64 and every logit is an
// fp64 sum in a fixed order, so identical rows give identical logits and
// exact ties are resolved by index, independent of scheduling.
//
// Three logit layouts, one selection:
//   route_small (T <= 64, decode): one workgroup per token; thread (e, ks)
//     sums the 16-byte chunks ks, ks+KS, ... of router row e against the
//     token row straight from global memory (all of a thread's loads issued
//     at once), then the KS partials are combined by a fixed butterfly.
//   route_screen (bf16, large T): bf16 MFMA screen with a rigorous error
//     bound, fp64 logits only for the experts that can still be selected.
//   route_tiled (fp32, large T): one workgroup per TT tokens; x and W chunks
//     are staged through LDS and thread (ks, e) keeps TT running logits, so
//     each router row is read once per TT tokens.
//   Logits out (optional, for the router's load statistics): the ranking
//   value of every (token, expert) pair rounded to fp32 -- exact for every
//   expert that could be selected; on the screen path the others get their
//   screen value, within the screen's bound of the exact one.
//   Selection (one wave per token): with at most 64 contenders, each lane
//     holds one and counts the contenders ranked above it (its rank), so the
//     k winners are known at once; with more, k rounds of a wave-wide argmax
//     (butterfly over (value, index)) pick them.  Either way the k
//     exponentials are then taken in parallel, one per lane, and summed in
//     rank order.
#include <atomic>

#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKC = 32;          // K elements per staged chunk (tiled)
constexpr int kMaxP = 256;       // experts per pass (tiled)
constexpr int kMaxE = 1024;
constexpr int kMaxDevices = 64;

template <typename In>
__device__ __forceinline__ void load8(const In* p, float* out);

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* out) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  out[0] = bf16lo(v.x); out[1] = bf16hi(v.x);
  out[2] = bf16lo(v.y); out[3] = bf16hi(v.y);
  out[4] = bf16lo(v.z); out[5] = bf16hi(v.z);
  out[6] = bf16lo(v.w); out[7] = bf16hi(v.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Raw 8-element chunk kept in registers until use (bf16: 16 bytes, fp32: 32).
template <typename In>
struct Raw8 {
  u32x4 v[sizeof(In) / 2];
  __device__ __forceinline__ void load(const In* p) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(In) / 2); ++i) v[i] = reinterpret_cast<const u32x4*>(p)[i];
  }
  __device__ __forceinline__ float get(int q) const {
    if constexpr (sizeof(In) == 2) {
      const uint32_t w = q < 2 ? v[0].x : q < 4 ? v[0].y : q < 6 ? v[0].z : v[0].w;
      return (q & 1) ? bf16hi(w) : bf16lo(w);
    } else {
      const u32x4& h = v[q >> 2];
      const uint32_t w = (q & 3) == 0 ? h.x : (q & 3) == 1 ? h.y : (q & 3) == 2 ? h.z : h.w;
      return __uint_as_float(w);
    }
  }
};

// (value, index) order of the ranking: larger value first, then lower index.
__device__ __forceinline__ bool better(double v, int e, double bv, int be) {
  return v > bv || (v == bv && e < be);
}

// The value an expert is ranked by: its fp64 logit plus the bias (if any);
// NaN ranks last.
__device__ __forceinline__ double rank_value(double logit, const float* __restrict__ bias,
                                             int e) {
  const double v = bias ? logit + (double)bias[e] : logit;
  return v != v ? -INFINITY : v;
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// LDS of one wave's selection: the k winners in rank order.
struct SelSlots {
  int e[64];
  double v[64];
};

// Lanes 0..k-1 hold the winners (value v, expert e) in rank order: write
// the ids and the renormalised weights exp(v_j - v_0) / sum_{i<k} exp(v_i - v_0),
// the sum taken in rank order.
__device__ __forceinline__ void emit_topk(double v, int e, int k, int32_t* __restrict__ idx_out,
                                          float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const double vmax = readlane_f64(v, 0);
  const double ex = lane < k ? exp(v - vmax) : 0.0;
  double wsum = 0.0;
  for (int j = 0; j < k; ++j) wsum += readlane_f64(ex, j);
  if (lane < k) {
    idx_out[lane] = e;
    w_out[lane] = (float)(ex / wsum);
  }
}

// Top-k of n <= 64 contenders held one per lane (lane i < n: value v, expert
// e; values are final ranking values).  Each lane's rank is the number of
// contenders ranked above it; ranks form a permutation of 0..n-1.
__device__ void topk_lanes(double v, int e, int n, int k, int32_t* __restrict__ idx_out,
                           float* __restrict__ w_out, SelSlots* sl) {
  const int lane = threadIdx.x & 63;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const double vj = readlane_f64(v, j);
    const int ej = __builtin_amdgcn_readlane(e, j);
    rank += better(vj, ej, v, e) ? 1 : 0;
  }
  if (lane < n && rank < k) {
    sl->e[rank] = e;
    sl->v[rank] = v;
  }
  // LDS operations of one wave complete in order: the reads below see the
  // writes above once they are issued
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const double vs = lane < k ? sl->v[lane] : 0.0;
  const int es = lane < k ? sl->e[lane] : 0;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  emit_topk(vs, es, k, idx_out, w_out);
}

// Top-k of the E final ranking values in LDS row `row` by one wave: k rounds
// of a wave-wide argmax over (value, index) (lane l owns experts l, l+64, ...;
// k <= 64, E <= 1024); lane j keeps the round-j winner.
__device__ void topk_rounds(const double* row, int E, int k, int32_t* __restrict__ idx_out,
                            float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  double my_v = 0.0;
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY;
    int be = 0x7fffffff;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      if ((taken >> m) & 1u) continue;
      const double v = row[e];
      if (better(v, e, bv, be)) {
        bv = v;
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // every lane now holds the winner (bv, be)
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == j) {
      my_v = bv;
      my_e = be;
    }
  }
  emit_topk(my_v, my_e, k, idx_out, w_out);
}

// Top-k of an LDS row of E final ranking values.
__device__ void topk_row(const double* row, int E, int k, int32_t* __restrict__ idx_out,
                         float* __restrict__ w_out, SelSlots* sl) {
  const int lane = threadIdx.x & 63;
  if (E <= 64) {
    topk_lanes(lane < E ? row[lane] : -INFINITY, lane, E, k, idx_out, w_out, sl);
  } else {
    topk_rounds(row, E, k, idx_out, w_out);
  }
}

// ------------------------------------------------------------ route_small
constexpr int kSmallThreads = 1024;

template <typename In>
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(
    const In* __restrict__ x, const In* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ logits_out,
    int64_t d, int E, int k, int KS) {
  __shared__ double logits[kMaxE];
  __shared__ SelSlots sl;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int per_pass = kSmallThreads / KS;
  const int ks = tid % KS;
  const int64_t nchunk = d / 8;
  const In* xr = x + t * d;
  // 8-element chunks of x and W loaded together per thread (one round of
  // loads covers rows of up to kSmallBatch*KS chunks)
  constexpr int kSmallBatch = sizeof(In) == 2 ? 12 : 6;
  for (int e0 = 0; e0 < E; e0 += per_pass) {
    const int e = e0 + tid / KS;
    double acc = 0.0;
    if (e < E) {
      const In* wr = Wr + (int64_t)e * d;
      // chunks ks, ks+KS, ... in order (chunks past the row read chunk 0
      // and are not used)
      for (int64_t c = ks; c < nchunk; c += kSmallBatch * KS) {
        Raw8<In> xv[kSmallBatch], wv[kSmallBatch];
#pragma unroll
        for (int u = 0; u < kSmallBatch; ++u) {
          const int64_t cc = c + u * KS;
          const int64_t ca = cc < nchunk ? cc : 0;
          xv[u].load(xr + ca * 8);
          wv[u].load(wr + ca * 8);
        }
#pragma unroll
        for (int u = 0; u < kSmallBatch; ++u) {
          if (c + u * KS < nchunk) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              acc = fma((double)xv[u].get(q), (double)wv[u].get(q), acc);
          }
        }
      }
    }
    // combine the KS partials of expert e (adjacent lanes) in a fixed order
    for (int off = 1; off < KS; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (ks == 0 && e < E) {
      logits[e] = rank_value(acc, bias, e);
      if (logits_out) logits_out[t * E + e] = (float)logits[e];
    }
  }
  __syncthreads();
  if (tid < 64) topk_row(logits, E, k, topk_idx + t * k, topk_w + t * k, &sl);
}

// ------------------------------------------------------------ route_tiled
template <int TT>
struct TiledSmem {
  static constexpr int kE = (TT == 16) ? 512 : 1024;
  double logits[TT][kE];         // 64 KB
  float w[kKC][kMaxP];           // staged router weights, transposed (32 KB)
  double xs[TT][kKC];            // staged token chunk (fp64)
  double part[kThreads][TT];     // k-split partial sums (32 KB at TT=16)
  SelSlots sl[kThreads / 64];
};

template <typename In, int TT>
__global__ __launch_bounds__(kThreads) void route_tiled_kernel(
    const In* __restrict__ x, const In* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ logits_out,
    int64_t T, int64_t d, int E, int k, int P) {
  __shared__ TiledSmem<TT> sm;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int KS = kThreads / P;     // k-splits per chunk
  const int e_loc = tid % P;
  const int ks = tid / P;

  for (int e0 = 0; e0 < E; e0 += P) {
    double acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0;

    for (int64_t k0 = 0; k0 < d; k0 += kKC) {
      // stage W[e0 .. e0+P, k0 .. k0+KC) transposed as float, 8 elements per piece
      const int pieces_w = P * (kKC / 8);
      for (int p = tid; p < pieces_w; p += kThreads) {
        const int row = p / (kKC / 8);
        const int part = p % (kKC / 8);
        const int64_t kk = k0 + part * 8;
        float v[8];
        if (e0 + row < E && kk < d) {
          load8<In>(Wr + (int64_t)(e0 + row) * d + kk, v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) sm.w[part * 8 + q][row] = v[q];
      }
      // stage x[t0 .. t0+TT, k0 .. k0+KC) as fp64
      const int pieces_x = TT * (kKC / 8);
      for (int p = tid; p < pieces_x; p += kThreads) {
        const int t = p / (kKC / 8);
        const int part = p % (kKC / 8);
        const int64_t kk = k0 + part * 8;
        float v[8];
        if (t0 + t < T && kk < d) {
          load8<In>(x + (t0 + t) * d + kk, v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) sm.xs[t][part * 8 + q] = (double)v[q];
      }
      __syncthreads();
      for (int kk = ks; kk < kKC; kk += KS) {
        const double w = (double)sm.w[kk][e_loc];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = fma(sm.xs[t][kk], w, acc[t]);
      }
      __syncthreads();
    }
    // add the k-split partials in fixed order
#pragma unroll
    for (int t = 0; t < TT; ++t) sm.part[tid][t] = acc[t];
    __syncthreads();
    if (ks == 0 && e0 + e_loc < E) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        double s = 0.0;
        for (int q = 0; q < KS; ++q) s += sm.part[q * P + e_loc][t];
        sm.logits[t][e0 + e_loc] = rank_value(s, bias, e0 + e_loc);
        if (logits_out && t0 + t < T)
          logits_out[(t0 + t) * E + e0 + e_loc] = (float)sm.logits[t][e0 + e_loc];
      }
    }
    __syncthreads();
  }

  const int wave = tid >> 6;
  for (int t = wave; t < TT; t += kThreads / 64) {
    if (t0 + t >= T) break;
    topk_row(sm.logits[t], E, k, topk_idx + (t0 + t) * k, topk_w + (t0 + t) * k,
             &sm.sl[wave]);
  }
}

// ----------------------------------------------------------- route_screen
// bf16, large T.  Exact fp64 logits of every (token, expert) pair cost
// 2*T*E*d fp64 flops; instead the experts are screened with bf16 MFMA and
// only the few that can still be in a token's top-k get an fp64 logit.
// One workgroup = 16 tokens x all experts, 8 waves.
//   1. MFMA screen.  K runs in steps of 64; a step's 16 token rows and the
//      pass's expert rows are copied to LDS (128 bytes per row, eight lanes
//      per row, so every group of four lanes reads one contiguous piece of
//      a line: reading sixteen rows per instruction in the MFMA's own lane
//      order is three times slower out of L2), and each wave reads its
//      operand fragments back from LDS: lane (j, kb) takes 16 consecutive
//      elements [16kb, +16) of row j and feeds their two halves to two
//      16x16x32 MFMAs (the sum over K does not depend on how K is split
//      between them).  The MFMA accumulates in fp32 over groups of 4 steps
//      (256 K elements); each group's sum is added to an fp64 total.  Every
//      bf16 product is exact in fp32, so the only error is the rounding
//      inside each group: at most 255 roundings of at most 2^-23 relative to
//      the running sum, bounded by 2^-15 * sum_i |x_i w_i| <= 2^-15 *
//      ||x_t|| * ||w_e|| (Cauchy-Schwarz).  The squared norms come from the
//      same fragments, as the diagonals of the Gram products W_blk W_blk^T
//      and X X^T (two more MFMAs each), accumulated the same way (relative
//      error <= 2^-15).  Screen logit L~ (+ bias), bound
//      b = 2^-14 * fac * ||x|| * ||w|| + 1e-30 (fac covers the norms' errors
//      and their rounding to fp32).
//   2. With lo = L~ - b, hi = L~ + b and tau = the k-th largest lo, an
//      expert whose hi < tau is below k others for certain; the rest are
//      the candidates (k of them, rarely a few more).
//   3. Candidates get their exact fp64 logit (same fixed summation order for
//      every expert, so identical rows still tie exactly), in batches of up
//      to 8 with the token row's chunks loaded once per batch.
//   4. Top-k over the candidates' exact logits.
// The result is the same selection and weights as the fp64-everywhere path.
// Precondition: finite inputs whose nonzero magnitudes lie in [2^-60, 2^60]
// (squares, products and partial sums stay normal and finite in fp32).
//
// Two kernels share this scheme: route_staged (E <= 256, operands staged
// through an LDS ring by direct global -> LDS copies) and route_direct (more
// experts: operands loaded straight into registers, 16 rows per load).
constexpr int kScreenTT = 16;                     // tokens per workgroup (MFMA rows)
constexpr int kScreenWaves = 8;
constexpr int kScreenThreads = 64 * kScreenWaves;
constexpr int kGroupSteps = 4;                    // 64-wide K steps per fp32 group
constexpr double kScreenRel = 6.103515625e-05;   // 2^-14
constexpr double kScreenFac = 1.0001220703125;   // 1 + 2^-13
constexpr int kExactPre = 3;                      // exact-phase chunk rounds in flight
constexpr int kStagedMaxE = 256;

// One staged K step: 16 token rows (ring X) and 128*NBW expert rows (ring
// W), 128 bytes each.
template <int NBW>
struct Staged {
  static constexpr int kWRows = 128 * NBW;
  static constexpr int kXStage = 16 * 128;
  static constexpr int kWStage = kWRows * 128;
  static constexpr int kStages = NBW == 1 ? 4 : 3;
  static constexpr int kCopies = 2 + kWRows / 8;                     // 1 KB copies per step
  static constexpr int kCpw = (kCopies + kScreenWaves - 1) / kScreenWaves;  // per wave
  static constexpr int kXBytes = kStages * kXStage;
  static constexpr int kWBytes = kStages * kWStage + 1024;           // + 1 KB for pad copies
  static constexpr int kRingBytes = kXBytes + kWBytes;
  static_assert((kStages - 1) * kCpw < 64, "vmcnt range");
};

// LDS layout of the screen kernels (bytes), sized by E at launch:
//   lg    [16][E] double    screen logits (+ bias), later exact logits / -inf
//   wn    [E]     float     ||w_e|| (rounded up)
//   xn    [16]    float     ||x_t|| (rounded up)
//   xp    [8][16] double    per-item partial ||x_t||^2 (K-split passes)
//   sl    [8]     SelSlots  per-wave selection slots
//   un: union { ring (staged kernel's copies of K steps),
//               part [8 items][16][16] double + wp [8 items][16] double
//               (K-split partials, passes of fewer than 8 blocks),
//               cand [8 waves][E] uint16 (candidate lists) }
struct ScreenLds {
  int64_t lg, wn, xn, xp, sl, un, total;
};
// split_parts: whether a pass can have fewer than 8 blocks (K-split partials
// then share the union).
__host__ __device__ constexpr ScreenLds screen_lds(int E, bool split_parts) {
  ScreenLds o{};
  o.lg = 0;
  o.wn = o.lg + (int64_t)kScreenTT * E * 8;
  o.xn = o.wn + ((int64_t)E * 4 + 15) / 16 * 16;
  o.xp = o.xn + kScreenTT * 4;
  o.sl = o.xp + 8 * 16 * 8;
  o.un = o.sl + (int64_t)kScreenWaves * sizeof(SelSlots);
  const int64_t part = split_parts ? 8 * 16 * 16 * 8 + 8 * 16 * 8 : 0;
  const int64_t cand = ((int64_t)kScreenWaves * E * 2 + 15) / 16 * 16;
  o.total = o.un + (part > cand ? part : cand);
  return o;
}
static_assert(screen_lds(kMaxE, true).total <= 160 * 1024, "direct screen LDS fits one CU");
static_assert(screen_lds(kStagedMaxE, false).total + Staged<2>::kRingBytes <= 160 * 1024,
              "staged screen LDS fits one CU");
static_assert(screen_lds(128, true).total + Staged<1>::kRingBytes <= 160 * 1024,
              "staged screen LDS fits one CU");

// fp32 value -> unsigned key with the same order (no NaN)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key >> 31) ? (key & 0x7fffffffu) : ~key);
}

// Element (r, r) of a 16x16 MFMA result, on the one lane that holds it:
// lane (j, kb) holds rows 4kb .. 4kb+3 of column j.
__device__ __forceinline__ bool holds_diag(int j, int kb) { return kb == (j >> 2); }

// Accumulators of one wave's items in one pass: screen logits and the Gram
// diagonals, fp32 within a group of steps and fp64 across groups.
template <int NBW>
struct ScreenAcc {
  f32x4 acc[NBW], accw[NBW], accx;
  double accD[NBW][4], wsqD[NBW][4], xsqD[4];
  __device__ __forceinline__ void zero() {
    accx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) xsqD[i] = 0.0;
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      acc[q] = accw[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) accD[q][i] = wsqD[q][i] = 0.0;
    }
  }
  // one 64-wide step: token fragments a0, a1; block q's fragments b0[q], b1[q]
  __device__ __forceinline__ void step(const u32x4& a0, const u32x4& a1, const u32x4* b0,
                                       const u32x4* b1) {
    accx = mfma16(a0, a0, accx);
    accx = mfma16(a1, a1, accx);
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      acc[q] = mfma16(a0, b0[q], acc[q]);
      acc[q] = mfma16(a1, b1[q], acc[q]);
      accw[q] = mfma16(b0[q], b0[q], accw[q]);
      accw[q] = mfma16(b1[q], b1[q], accw[q]);
    }
  }
  __device__ __forceinline__ void flush() {
#pragma unroll
    for (int i = 0; i < 4; ++i) xsqD[i] += (double)accx[i];
    accx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        accD[q][i] += (double)acc[q][i];
        wsqD[q][i] += (double)accw[q][i];
      }
      acc[q] = accw[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Pointers into the screen kernels' LDS.
struct ScreenSmem {
  double* lg;
  float* wn;
  float* xn;
  double* xp;
  SelSlots* sls;
  double* part;
  double* wp;
  uint16_t* cand;
  unsigned char* ring;
  __device__ ScreenSmem(unsigned char* smem, const ScreenLds& L, unsigned char* ring_ = nullptr) {
    lg = reinterpret_cast<double*>(smem + L.lg);
    wn = reinterpret_cast<float*>(smem + L.wn);
    xn = reinterpret_cast<float*>(smem + L.xn);
    xp = reinterpret_cast<double*>(smem + L.xp);
    sls = reinterpret_cast<SelSlots*>(smem + L.sl);
    part = reinterpret_cast<double*>(smem + L.un);
    wp = reinterpret_cast<double*>(smem + L.un + 8 * 16 * 16 * 8);
    cand = reinterpret_cast<uint16_t*>(smem + L.un);
    ring = ring_;
  }
};

// End of a screen pass: the items' screen logits (+ bias), ||w_e|| and (first
// pass) ||x_t|| go to LDS; K-split items are added in split order.  Every
// thread of the workgroup calls it; it ends with a barrier.
template <int NBW>
__device__ void screen_pass_store(const ScreenAcc<NBW>& A, const ScreenSmem& S,
                                  const float* __restrict__ bias, int E, int e0, int nb, int KS,
                                  const bool* live, const int* blk, bool xnorm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kb = lane >> 4;
  const bool diag = holds_diag(j, kb);
  // lane holds D[4kb + i][j] of each block: token 4kb+i, expert 16*blk+j;
  // the Gram diagonals (squared norms) sit on the lanes with kb = j/4
  const int dq = j & 3;
  double wsq[NBW];
#pragma unroll
  for (int q = 0; q < NBW; ++q)
    wsq[q] = dq == 0 ? A.wsqD[q][0] : dq == 1 ? A.wsqD[q][1] : dq == 2 ? A.wsqD[q][2] : A.wsqD[q][3];
  const double xsq = dq == 0 ? A.xsqD[0] : dq == 1 ? A.xsqD[1] : dq == 2 ? A.xsqD[2] : A.xsqD[3];
  if (KS == 1) {
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int e = e0 + 16 * blk[q] + j;
      if (live[q] && e < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S.lg[(4 * kb + i) * E + e] = rank_value(A.accD[q][i], bias, e);
        if (diag) S.wn[e] = __double2float_ru(sqrt(wsq[q]));
      }
    }
    if (xnorm && diag) S.xp[0 * 16 + j] = xsq;
  }
  __syncthreads();  // part / wp / xp (K split) are written next; lg readers wait
  if (KS > 1) {
    const int it = wave;  // one item per wave
    if (live[0]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S.part[(it * 16 + 4 * kb + i) * 16 + j] = A.accD[0][i];
      if (diag) {
        S.wp[it * 16 + j] = wsq[0];
        if (xnorm) S.xp[it * 16 + j] = xsq;
      }
    }
    __syncthreads();
    // add the K-split partials in split order; items blk + nb*ks
    for (int o = tid; o < nb * 256; o += kScreenThreads) {
      const int b = o / 256, rr = (o / 16) % 16, c = o % 16;
      const int e = e0 + 16 * b + c;
      double sacc = 0.0;
      for (int q = 0; q < KS; ++q) sacc += S.part[((b + nb * q) * 16 + rr) * 16 + c];
      if (e < E) S.lg[rr * E + e] = rank_value(sacc, bias, e);
    }
    if (tid < nb * 16) {
      const int b = tid / 16, c = tid % 16;
      double sq = 0.0;
      for (int q = 0; q < KS; ++q) sq += S.wp[(b + nb * q) * 16 + c];
      if (e0 + tid < E) S.wn[e0 + tid] = __double2float_ru(sqrt(sq));
    }
  }
  if (e0 == 0 && tid < 16) {
    // ||x_t||^2: items with block 0 cover every K step once (split order)
    double sq = 0.0;
    for (int q = 0; q < KS; ++q) sq += S.xp[(nb * q) * 16 + tid];
    S.xn[tid] = __double2float_ru(sqrt(sq));
  }
  __syncthreads();
}

// Exact fp64 logits of candidates c0 .. c0+CB-1 of one token (CB <= 8): lane
// l sums the 16-byte chunks l, l+64, ... of the row in order, a ring of
// kExactPre chunk rounds of loads in flight; the CB sums are then reduced
// over the 64 lanes in a fixed order (halving exchanges leave lane l with
// candidate u = l*CB/64, then a butterfly over the 64/CB lanes sharing it;
// pairs are always formed over lane bit 5, then 4, ..., then 0, so every
// candidate's sum has the same rounding).  Lane u < CB returns the sum of
// candidate c0 + u.
template <int CB, int PRE = kExactPre>
__device__ __forceinline__ double exact_batch(const bf16_t* __restrict__ xt,
                                              const bf16_t* __restrict__ Wr,
                                              const uint16_t* cands, int c0, int ncand,
                                              int64_t d) {
  const int lane = threadIdx.x & 63;
  const int64_t n8 = d / 8;
  const int64_t nr = (n8 + 63) / 64;  // chunk rounds
  double a[CB];
  const bf16_t* wr[CB];
#pragma unroll
  for (int u = 0; u < CB; ++u) {
    a[u] = 0.0;
    const int ci = c0 + u < ncand ? c0 + u : ncand - 1;
    wr[u] = Wr + (int64_t)cands[ci] * d;
  }
  struct ExRegs {
    u32x4 xv, wv[CB];
  };
  ExRegs rr[PRE];
  // rounds past the row read chunk 0 and add nothing
  auto eld = [&](int64_t r, ExRegs& g) {
    const int64_t ch = 64 * r + lane;
    const int64_t o = ch < n8 ? ch * 8 : 0;
    g.xv = ldg16(xt + o);
#pragma unroll
    for (int u = 0; u < CB; ++u) g.wv[u] = ldg16(wr[u] + o);
  };
  auto eacc = [&](int64_t r, const ExRegs& g) {
    if (64 * r + lane >= n8) return;
    const uint32_t xw[4] = {g.xv.x, g.xv.y, g.xv.z, g.xv.w};
    double xd[8];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      xd[2 * h] = (double)bf16lo(xw[h]);
      xd[2 * h + 1] = (double)bf16hi(xw[h]);
    }
#pragma unroll
    for (int u = 0; u < CB; ++u) {
      const uint32_t w[4] = {g.wv[u].x, g.wv[u].y, g.wv[u].z, g.wv[u].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        a[u] = fma(xd[2 * h], (double)bf16lo(w[h]), a[u]);
        a[u] = fma(xd[2 * h + 1], (double)bf16hi(w[h]), a[u]);
      }
    }
  };
#pragma unroll
  for (int q = 0; q < PRE; ++q) eld(q, rr[q]);
  for (int64_t r0 = 0; r0 < nr; r0 += PRE) {
#pragma unroll
    for (int q = 0; q < PRE; ++q) {
      eacc(r0 + q, rr[q]);
      eld(r0 + q + PRE, rr[q]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // halving exchanges over lane bits 5, 4, 3 (as many as CB needs)
  constexpr int LB = CB == 8 ? 3 : CB == 4 ? 2 : CB == 2 ? 1 : 0;
  double v = a[0];
  if constexpr (LB >= 1) {
    double b[CB / 2];
    const bool h = lane & 32;
#pragma unroll
    for (int i = 0; i < CB / 2; ++i) {
      const double send = h ? a[i] : a[i + CB / 2];
      const double keep = h ? a[i + CB / 2] : a[i];
      b[i] = keep + __shfl_xor(send, 32, 64);
    }
    if constexpr (LB >= 2) {
      double c[CB / 4];
      const bool h2 = lane & 16;
#pragma unroll
      for (int i = 0; i < CB / 4; ++i) {
        const double send = h2 ? b[i] : b[i + CB / 4];
        const double keep = h2 ? b[i + CB / 4] : b[i];
        c[i] = keep + __shfl_xor(send, 16, 64);
      }
      if constexpr (LB >= 3) {
        const bool h3 = lane & 8;
        const double send = h3 ? c[0] : c[1];
        const double keep = h3 ? c[1] : c[0];
        v = keep + __shfl_xor(send, 8, 64);
      } else {
        v = c[0];
      }
    } else {
      v = b[0];
    }
  }
  // butterfly over the lanes that share a candidate (bits below 6 - LB)
#pragma unroll
  for (int off = 32 >> LB; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  // candidate u's sum is on lanes u*64/CB ..; lane u < CB takes it
  return __shfl(v, lane < CB ? lane * (64 / CB) : 0, 64);
}

// Steps 2-4 for the workgroup's TT tokens, one wave per token, once the
// screen logits and norms are in LDS (and the ring is no longer in use).  M:
// experts per lane, at least ceil(E / 64).
template <int M, int TT = kScreenTT, int MaxCB = 8, int PRE = kExactPre>
__device__ void screen_select(const ScreenSmem& S, const bf16_t* __restrict__ x,
                              const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
                              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                              float* __restrict__ logits_out, int64_t T, int64_t d, int E,
                              int k, int64_t t0) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint16_t* mycand = S.cand + wave * E;
  SelSlots* sl = S.sls + wave;
  const double rel = kScreenRel * kScreenFac;
  for (int tl = wave; tl < TT; tl += kScreenWaves) {
    const int64_t t = t0 + tl;
    if (t >= T) break;
    double* row = S.lg + (int64_t)tl * E;
    const double xn = (double)S.xn[tl];
    // tau: a value at most the k-th largest lower bound lo = L~ - b, so the
    // test below keeps every expert that can be selected.  lo is rounded
    // down to fp32 and mapped to an order-preserving 32-bit key; a radix
    // selection over the top 16 bits of the keys (bit by bit from the top,
    // keep the bit if at least k keys have top bits >= the prefix with it
    // set) ends on exactly the top 16 bits of the k-th largest key (a larger
    // prefix would put k keys above it), and tau is that prefix with the low
    // bits cleared: within 2^-7 relative of the k-th largest lo.
    uint32_t key[M];
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const int e = lane + 64 * q;
      key[q] = 0u;  // below every real key
      if (e < E) {
        double lo = row[e] - (rel * xn * (double)S.wn[e] + 1e-30);
        if (lo != lo) lo = -INFINITY;
        key[q] = order_key(__double2float_rd(lo)) >> 16;
      }
    }
    uint32_t prefix = 0u;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = prefix | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int q = 0; q < M; ++q) cnt += __popcll(__ballot(key[q] >= c));
      if (cnt >= k) prefix = c;
    }
    const double tau = (double)key_value(prefix << 16);
    // candidates: hi >= tau, listed in expert order
    int ncand = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      bool c = false;
      if (e < E) c = !(row[e] + (rel * xn * (double)S.wn[e] + 1e-30) < tau);
      // logits asked for: the screen value of every expert ruled out (the
      // candidates' exact values follow below)
      if (logits_out && e < E && !c) logits_out[t * E + e] = (float)row[e];
      const uint64_t mk = __ballot(c);
      if (c) mycand[ncand + __popcll(mk & ((1ull << lane) - 1ull))] = (uint16_t)e;
      ncand += __popcll(mk);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (ncand > 64) {
      // many candidates (degenerate inputs): exact logits go back into the
      // row, every non-candidate drops out, and the row is ranked in rounds
      for (int e = lane; e < E; e += 64) row[e] = -INFINITY;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // exact fp64 logits of the candidates, in batches of 8, 4, 2 or 1
    const bf16_t* xt = x + t * d;
    double my_v = -INFINITY;
    int my_e = 0;
    for (int c0 = 0; c0 < ncand;) {
      const int left = ncand - c0;
      const int cb = (left >= 8 && MaxCB >= 8) ? 8 : (left >= 4 && MaxCB >= 4) ? 4
                     : left >= 2 ? 2 : 1;
      double got;  // lane u < cb: candidate c0 + u
      if (MaxCB >= 8 && cb == 8) got = exact_batch<8, PRE>(xt, Wr, mycand, c0, ncand, d);
      else if (MaxCB >= 4 && cb == 4) got = exact_batch<4, PRE>(xt, Wr, mycand, c0, ncand, d);
      else if (cb == 2) got = exact_batch<2, PRE>(xt, Wr, mycand, c0, ncand, d);
      else got = exact_batch<1, PRE>(xt, Wr, mycand, c0, ncand, d);
      if (ncand > 64) {
        if (lane < cb) {
          const int e = mycand[c0 + lane];
          row[e] = rank_value(got, bias, e);
          if (logits_out) logits_out[t * E + e] = (float)row[e];
        }
      } else {
        // lane c of the list holds candidate c
        const int want = lane - c0;
        const double v = __shfl(got, want >= 0 && want < cb ? want : 0, 64);
        if (want >= 0 && want < cb) {
          my_e = mycand[lane];
          my_v = rank_value(v, bias, my_e);
          if (logits_out) logits_out[t * E + my_e] = (float)my_v;
        }
      }
      c0 += cb;
    }
    if (ncand <= 64) {
      topk_lanes(my_v, my_e, ncand, k, topk_idx + t * k, topk_w + t * k, sl);
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      topk_rounds(row, E, k, topk_idx + t * k, topk_w + t * k);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Items of a pass: item i = wave + 8q is block i % nb, K split i / nb.
template <int NBW>
struct PassItems {
  int nb, KS, ks;
  bool live[NBW];
  int blk[NBW];
  bool xnorm;
  __device__ PassItems(int E, int e0, int wave) {
    nb = min(8 * NBW, (E - e0 + 15) / 16);
    KS = nb >= 8 ? 1 : 8 / nb;
    const int nitem = nb * KS;
    ks = 0;
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int it = wave + 8 * q;
      live[q] = it < nitem;
      blk[q] = live[q] ? it % nb : 0;
      if (q == 0) ks = live[0] ? it / nb : 0;
    }
    // items of block 0 (together covering every step once) keep ||x||^2
    xnorm = e0 == 0 && live[0] && blk[0] == 0;
  }
};

// ------------------------------------------------------------ route_staged
template <int NBW>
__global__ __launch_bounds__(kScreenThreads, 1) void route_staged_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ logits_out,
    int64_t T, int64_t d, int E, int k) {
  using SG = Staged<NBW>;
  // the rings are LDS objects of their own: with more than one LDS object
  // the compiler tags every LDS access with the object it touches, and the
  // fragment reads then need not wait for the copies in flight (which carry
  // no tag, their address being opaque); the kernel's own vmcnt waits and
  // barriers order each read after the copies it needs
  __shared__ __attribute__((aligned(1024))) unsigned char ringX[SG::kXBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char ringW[SG::kWBytes];
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  // NBW == 2 runs one pass of more than 128 experts: never a K split
  const ScreenLds L = screen_lds(E, NBW == 1);
  const ScreenSmem S(smem, L);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kScreenTT;
  const uint32_t rowb = (uint32_t)(d * 2);          // bytes per row
  const int64_t nsteps = (d + 63) / 64;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)(uint32_t)(T * d * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)Wr, 0, (int)(uint32_t)(E * d * 2), kRsrcWord3);
  // the rings' LDS addresses as integers for the copies, kept apart from
  // the pointer arithmetic of the fragment reads
  uint32_t ringx_i = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringX;
  uint32_t ringw_i = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringW;
  asm("" : "+s"(ringx_i), "+s"(ringw_i));
  const uint32_t pad_dst = ringw_i + SG::kStages * SG::kWStage;

  for (int e0 = 0; e0 < E; e0 += 128 * NBW) {
    const PassItems<NBW> P(E, e0, wave);
    // copy plan: copy i = wave + 8c (c < kCpw) moves stage rows 8i .. 8i+7,
    // lane l: row 8i + l/8, LDS chunk l%8, which holds the row's 16-byte
    // chunk (l%8) ^ (row%8) (so that the fragment reads below, 16 rows at a
    // time, hit 8 distinct chunk positions).  Rows < 16 are tokens (the
    // padding rows past T repeat the last token), the rest experts e0 + ...
    // (past E: out of range, zero).  Copies i >= kCopies are padding: they
    // land in a spare 1 KB and move nothing.
    uint32_t base[SG::kCpw], kch[SG::kCpw], dst[SG::kCpw];
#pragma unroll
    for (int c = 0; c < SG::kCpw; ++c) {
      const int i = wave + 8 * c;
      const int r = 8 * i + (lane >> 3);  // stage row: tokens, then experts
      kch[c] = (uint32_t)(((lane & 7) ^ (r & 7)) * 16);
      uint32_t b = kOOB;
      if (i < SG::kCopies) {
        if (r < 16) {
          const int64_t t = t0 + r < T ? t0 + r : T - 1;
          b = (uint32_t)t * rowb;
        } else if (e0 + r - 16 < E) {
          b = (uint32_t)(e0 + r - 16) * rowb;
        }
      }
      base[c] = b;
      // byte offset of the copy's 8 rows inside its ring's stage
      dst[c] = i < 2 ? (uint32_t)(8 * i) * 128 : (uint32_t)(8 * (i - 2)) * 128;
    }
    auto issue = [&](int stage, int64_t s) {
      const uint32_t koff = (uint32_t)(s * 128);
#pragma unroll
      for (int c = 0; c < SG::kCpw; ++c) {
        const int i = wave + 8 * c;
        const uint32_t o = (base[c] != kOOB && koff + kch[c] < rowb) ? base[c] + koff + kch[c]
                                                                     : kOOB;
        if (i < 2)
          copy16(rx, o, ringx_i + (uint32_t)stage * SG::kXStage + dst[c]);
        else if (i < SG::kCopies)
          copy16(rw, o, ringw_i + (uint32_t)stage * SG::kWStage + dst[c]);
        else
          copy16(rw, kOOB, pad_dst);
      }
    };
    // fragment offsets inside a stage: row j (tokens) and 16*blk[q] + j
    // (experts), chunks 2kb and 2kb+1, swizzled by j%8 (= row%8 of both)
    const uint32_t f0 = (uint32_t)(((2 * kb) ^ (j & 7)) * 16);
    const uint32_t f1 = (uint32_t)(((2 * kb + 1) ^ (j & 7)) * 16);
    uint32_t fb[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) fb[q] = (uint32_t)(16 * P.blk[q] + j) * 128;

    ScreenAcc<NBW> A;
    A.zero();
    // ring prologue: steps 0 .. kStages-1
#pragma unroll
    for (int q = 0; q < SG::kStages; ++q) issue(q, q);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((SG::kStages - 1) * SG::kCpw) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int stage = 0;
    int64_t mine = 0;  // steps this wave has accumulated in the current group
    for (int64_t s = 0; s < nsteps; ++s) {
      if (P.live[0] && (P.KS == 1 || s % P.KS == P.ks)) {
        const unsigned char* sx = ringX + (uint32_t)stage * SG::kXStage;
        const unsigned char* sw = ringW + (uint32_t)stage * SG::kWStage;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(sx + (uint32_t)j * 128 + f0);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(sx + (uint32_t)j * 128 + f1);
        u32x4 b0[NBW], b1[NBW];
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
          b0[q] = *reinterpret_cast<const u32x4*>(sw + fb[q] + f0);
          b1[q] = *reinterpret_cast<const u32x4*>(sw + fb[q] + f1);
        }
        A.step(a0, a1, b0, b1);
        if (++mine == kGroupSteps) {
          A.flush();
          mine = 0;
        }
      }
      // step s+1 has landed (this wave's copies, then everyone's: a plain
      // s_barrier), and every wave's reads of step s are complete (lgkmcnt(0)
      // before the barrier), so step s's stage can be refilled
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((SG::kStages - 2) * SG::kCpw)
                   : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue(stage, s + SG::kStages);
      stage = stage + 1 == SG::kStages ? 0 : stage + 1;
    }
    A.flush();
    // drain the copies still in flight before the ring's LDS is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    screen_pass_store<NBW>(A, S, bias, E, e0, P.nb, P.KS, P.live, P.blk, P.xnorm);
  }
  // experts per lane of the selection: 1, 2, 4 or 16
  if (E <= 64) screen_select<1>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else if (E <= 128) screen_select<2>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else if (E <= 256) screen_select<4>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else screen_select<16>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
}

// ------------------------------------------------------------ route_direct
// Loads of one 64-wide K step: chunks c0 = 8s + 2kb and c0+1 of the token
// row (A) and of each block's expert row (B), straight into registers.
template <int NBW>
struct StepRegs {
  u32x4 a0, a1, b0[NBW], b1[NBW];
};

template <int NBW>
__global__ __launch_bounds__(kScreenThreads, 1) void route_direct_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ logits_out,
    int64_t T, int64_t d, int E, int k) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const ScreenLds L = screen_lds(E, true);
  const ScreenSmem S(smem, L);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kScreenTT;
  const int64_t tj = t0 + j < T ? t0 + j : T - 1;  // padding rows repeat the last token
  const bf16_t* xa = x + tj * d;
  const int64_t n8 = d / 8;          // 8-element chunks per row
  const int64_t nfull = n8 / 8;      // K steps with all 64 elements inside the row
  const int64_t nsteps = (n8 + 7) / 8;

  for (int e0 = 0; e0 < E; e0 += 128 * NBW) {
    const PassItems<NBW> P(E, e0, wave);
    const bf16_t* wb[NBW];
#pragma unroll
    for (int q = 0; q < NBW; ++q) {
      const int e = e0 + 16 * P.blk[q] + j;
      wb[q] = Wr + (int64_t)(e < E ? e : E - 1) * d;
    }
    // a wave with fewer live blocks runs the missing ones on its first
    // block's rows (the same lines, served by L1) and drops the result: no
    // load depends on a branch, so the wait counters keep the ring in flight
#pragma unroll
    for (int q = 1; q < NBW; ++q)
      if (!P.live[q]) wb[q] = wb[0];
    const int ks = P.ks, KS = P.KS;
    ScreenAcc<NBW> A;
    A.zero();
    // step s is loaded from chunk 0 where it runs past the row; only the
    // last step can, and its chunks past the row are zeroed before use
    auto ld = [&](int64_t s, StepRegs<NBW>& r) {
      const int64_t c0 = 8 * s + 2 * kb;
      const int64_t o0 = c0 < n8 ? c0 * 8 : 0, o1 = c0 + 1 < n8 ? (c0 + 1) * 8 : 0;
      r.a0 = ldg16(xa + o0);
      r.a1 = ldg16(xa + o1);
#pragma unroll
      for (int q = 0; q < NBW; ++q) {
        r.b0[q] = ldg16(wb[q] + o0);
        r.b1[q] = ldg16(wb[q] + o1);
      }
    };
    auto mm = [&](int64_t s, StepRegs<NBW>& r, bool ragged) {
      if (ragged) {
        const int64_t c0 = 8 * s + 2 * kb;
        const bool ok0 = c0 < n8, ok1 = c0 + 1 < n8;
        r.a0 = zero_unless(ok0, r.a0);
        r.a1 = zero_unless(ok1, r.a1);
#pragma unroll
        for (int q = 0; q < NBW; ++q) {
          r.b0[q] = zero_unless(ok0, r.b0[q]);
          r.b1[q] = zero_unless(ok1, r.b1[q]);
        }
      }
      A.step(r.a0, r.a1, r.b0, r.b1);
    };
    if (P.live[0]) {
      // this wave's steps ks, ks + KS, ...: a ring of kGroupSteps register
      // sets keeps that many steps' loads in flight; each pass of the ring
      // is one fp32 accumulation group.  Groups whose steps all lie inside
      // the row run without masking; the rest (at most one group and a
      // partial one, padded with steps past the row) run masked after them.
      // The ring's loads past the last group read chunk 0 and are not used.
      const int64_t nmine = nsteps > ks ? (nsteps - ks + KS - 1) / KS : 0;
      const int64_t ngroups = (nmine + kGroupSteps - 1) / kGroupSteps;
      const int64_t nmine_full = nfull > ks ? (nfull - ks + KS - 1) / KS : 0;
      const int64_t gfull = nmine_full / kGroupSteps;
      StepRegs<NBW> rs[kGroupSteps];
#pragma unroll
      for (int q = 0; q < kGroupSteps; ++q) ld(ks + q * KS, rs[q]);
      for (int64_t g = 0; g < gfull; ++g) {
#pragma unroll
        for (int q = 0; q < kGroupSteps; ++q) {
          const int64_t st = ks + (g * kGroupSteps + q) * KS;
          mm(st, rs[q], false);
          ld(st + kGroupSteps * KS, rs[q]);
          // keep each refill right after the step that frees its registers
          __builtin_amdgcn_sched_barrier(0);
        }
        A.flush();
      }
      for (int64_t g = gfull; g < ngroups; ++g) {
#pragma unroll
        for (int q = 0; q < kGroupSteps; ++q) {
          const int64_t st = ks + (g * kGroupSteps + q) * KS;
          mm(st, rs[q], true);
          ld(st + kGroupSteps * KS, rs[q]);
          __builtin_amdgcn_sched_barrier(0);
        }
        A.flush();
      }
    }
    screen_pass_store<NBW>(A, S, bias, E, e0, P.nb, P.KS, P.live, P.blk, P.xnorm);
  }
  // experts per lane of the selection: 1, 2, 4 or 16
  if (E <= 64) screen_select<1>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else if (E <= 128) screen_select<2>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else if (E <= 256) screen_select<4>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
  else screen_select<16>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
}

// ------------------------------------------------------------ route_split
// bf16, large T, with a scratch buffer for the partial sums: the screen of
// route_staged as a K-split product over tiles of 16*NTB tokens x 16*NEB
// experts (route_part), then the selection, one wave per token (route_pick).
// route_staged copies every expert row into LDS once per 16 tokens; here
// once per 16*NTB, and the K split gives every CU a tile when T / (16*NTB)
// tiles alone would not.  The arithmetic is the screen's: fp32 MFMA sums over
// groups of 4 K steps of 64 (restarted at the start of each split), each
// group added to an fp64 total; the splits' fp64 totals are added in split
// order.  The screen bound therefore holds unchanged.
//   part [SK][T][E] double   screen logits of split s (no bias)
//   xsq  [SK][T]    double   ||x_t||^2 of split s (Gram diagonal)
//   wsq  [SK][E]    double   ||w_e||^2 of split s
template <int NTB, int NEB, int WT, int WE>
struct PartCfg {
  static constexpr int kNWE = NEB / WE;  // wave columns (expert groups)
  static_assert(NTB % WT == 0 && NEB % WE == 0 && (NTB / WT) * kNWE == kScreenWaves,
                "one wave tile per wave");
  static constexpr int kXRows = 16 * NTB, kWRows = 16 * NEB;
  static constexpr int kXStage = kXRows * 128, kWStage = kWRows * 128;
  static constexpr int kXCopies = kXRows / 8;
  static constexpr int kCopies = (kXRows + kWRows) / 8;  // 1 KB copies per K step
  static constexpr int kCpw = (kCopies + kScreenWaves - 1) / kScreenWaves;
  static constexpr int kStages = (kXStage + kWStage) * 4 <= 112 * 1024 ? 4 : 3;
  static_assert((kStages - 1) * kCpw < 64, "vmcnt range");
};

template <int NTB, int NEB, int WT, int WE>
__global__ __launch_bounds__(kScreenThreads, 1) void route_part_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, double* __restrict__ part,
    double* __restrict__ xsq, double* __restrict__ wsq, int64_t T, int64_t d, int E, int SK,
    int ntiles) {
  using C = PartCfg<NTB, NEB, WT, WE>;
  // two LDS objects (see route_staged): the fragment reads need not wait
  // for copies in flight; the vmcnt waits and barriers order them
  __shared__ __attribute__((aligned(1024))) unsigned char ringX[C::kStages * C::kXStage];
  __shared__ __attribute__((aligned(1024))) unsigned char ringW[C::kStages * C::kWStage + 1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, kb = lane >> 4;
  // workgroup -> (token tile, split): consecutive workgroups go to the 8
  // XCDs in turn; split s = xcd % SK, so the tiles of one split, which read
  // the same columns of W, share an XCD's L2
  const int xcd = (int)(blockIdx.x % 8u), slot = (int)(blockIdx.x / 8u);
  const int s = xcd % SK;
  const int tile = xcd / SK + (8 / SK) * slot;
  if (tile >= ntiles) return;
  const int64_t t0 = (int64_t)tile * C::kXRows;
  const int64_t nsteps = (d + 63) / 64;
  const int64_t per = (nsteps + SK - 1) / SK;
  const int64_t s0 = (int64_t)s * per;
  const int64_t s1 = s0 + per < nsteps ? s0 + per : nsteps;  // may be <= s0: an empty split
  const uint32_t rowb = (uint32_t)(d * 2);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, 0, (int)(uint32_t)(T * d * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)Wr, 0, (int)(uint32_t)(E * d * 2), kRsrcWord3);
  uint32_t ringx_i = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringX;
  uint32_t ringw_i = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)ringW;
  asm("" : "+s"(ringx_i), "+s"(ringw_i));
  const uint32_t pad_dst = ringw_i + C::kStages * C::kWStage;

  // copy plan (route_staged's): copy i = wave + 8c moves stage rows 8i ..
  // 8i+7, lane l row 8i + l/8, LDS chunk l%8 holding the row's chunk
  // (l%8) ^ (row%8).  Rows < 16*NTB are tokens (past T: the last token
  // again), the rest experts (past E: out of range, zero).
  uint32_t base[C::kCpw], kch[C::kCpw], dst[C::kCpw];
#pragma unroll
  for (int c = 0; c < C::kCpw; ++c) {
    const int i = wave + 8 * c;
    const int r = 8 * i + (lane >> 3);
    kch[c] = (uint32_t)(((lane & 7) ^ (r & 7)) * 16);
    uint32_t b = kOOB;
    if (i < C::kXCopies) {
      const int64_t t = t0 + r < T ? t0 + r : T - 1;
      b = (uint32_t)t * rowb;
    } else if (i < C::kCopies && r - C::kXRows < E) {
      b = (uint32_t)(r - C::kXRows) * rowb;
    }
    base[c] = b;
    dst[c] = i < C::kXCopies ? (uint32_t)(8 * i) * 128 : (uint32_t)(8 * (i - C::kXCopies)) * 128;
  }
  auto issue = [&](int stage, int64_t st) {
    const uint32_t koff = (uint32_t)(st * 128);
    const bool live = st < s1;
#pragma unroll
    for (int c = 0; c < C::kCpw; ++c) {
      const int i = wave + 8 * c;
      const uint32_t o =
          (live && base[c] != kOOB && koff + kch[c] < rowb) ? base[c] + koff + kch[c] : kOOB;
      if (i < C::kXCopies)
        copy16(rx, o, ringx_i + (uint32_t)stage * C::kXStage + dst[c]);
      else if (i < C::kCopies)
        copy16(rw, o, ringw_i + (uint32_t)stage * C::kWStage + dst[c]);
      else
        copy16(rw, kOOB, pad_dst);
    }
  };
  // this wave's tile: token blocks tg*WT + p, expert blocks eg*WE + q
  const int tg = wave / C::kNWE, eg = wave % C::kNWE;
  const uint32_t f0 = (uint32_t)(((2 * kb) ^ (j & 7)) * 16);
  const uint32_t f1 = (uint32_t)(((2 * kb + 1) ^ (j & 7)) * 16);
  const bool xnorm = eg == 0;                // every tile: ||x||^2 of its tokens
  const bool wnorm = tile == 0 && tg == 0;   // tile 0: ||w||^2 of every expert

  f32x4 acc[WT][WE], accx[WT], accw[WE];
  double accD[WT][WE][4], xsqD[WT][4], wsqD[WE][4];
#pragma unroll
  for (int p = 0; p < WT; ++p) {
    accx[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) xsqD[p][i] = 0.0;
#pragma unroll
    for (int q = 0; q < WE; ++q) {
      acc[p][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) accD[p][q][i] = 0.0;
    }
  }
#pragma unroll
  for (int q = 0; q < WE; ++q) {
    accw[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) wsqD[q][i] = 0.0;
  }
  auto flush = [&]() {
#pragma unroll
    for (int p = 0; p < WT; ++p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xsqD[p][i] += (double)accx[p][i];
      accx[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < WE; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) accD[p][q][i] += (double)acc[p][q][i];
        acc[p][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int q = 0; q < WE; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) wsqD[q][i] += (double)accw[q][i];
      accw[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };

#pragma unroll
  for (int q = 0; q < C::kStages; ++q) issue(q, s0 + q);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((C::kStages - 1) * C::kCpw) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int stage = 0, mine = 0;
  for (int64_t st = s0; st < s1; ++st) {
    const unsigned char* sx = ringX + (uint32_t)stage * C::kXStage;
    const unsigned char* sw = ringW + (uint32_t)stage * C::kWStage;
    u32x4 a0[WT], a1[WT], b0[WE], b1[WE];
#pragma unroll
    for (int p = 0; p < WT; ++p) {
      const uint32_t ro = (uint32_t)(16 * (tg * WT + p) + j) * 128;
      a0[p] = *reinterpret_cast<const u32x4*>(sx + ro + f0);
      a1[p] = *reinterpret_cast<const u32x4*>(sx + ro + f1);
    }
#pragma unroll
    for (int q = 0; q < WE; ++q) {
      const uint32_t ro = (uint32_t)(16 * (eg * WE + q) + j) * 128;
      b0[q] = *reinterpret_cast<const u32x4*>(sw + ro + f0);
      b1[q] = *reinterpret_cast<const u32x4*>(sw + ro + f1);
    }
#pragma unroll
    for (int p = 0; p < WT; ++p) {
#pragma unroll
      for (int q = 0; q < WE; ++q) {
        acc[p][q] = mfma16(a0[p], b0[q], acc[p][q]);
        acc[p][q] = mfma16(a1[p], b1[q], acc[p][q]);
      }
    }
    if (xnorm) {
#pragma unroll
      for (int p = 0; p < WT; ++p) {
        accx[p] = mfma16(a0[p], a0[p], accx[p]);
        accx[p] = mfma16(a1[p], a1[p], accx[p]);
      }
    }
    if (wnorm) {
#pragma unroll
      for (int q = 0; q < WE; ++q) {
        accw[q] = mfma16(b0[q], b0[q], accw[q]);
        accw[q] = mfma16(b1[q], b1[q], accw[q]);
      }
    }
    if (++mine == kGroupSteps) {
      flush();
      mine = 0;
    }
    // step st+1 has landed everywhere and every read of step st is done:
    // refill step st's stage
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((C::kStages - 2) * C::kCpw) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(stage, st + C::kStages);
    stage = stage + 1 == C::kStages ? 0 : stage + 1;
  }
  flush();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane (j, kb) holds D[4kb + i][j] of every block pair; the Gram
  // diagonals sit on the lanes with kb = j/4, element j%4
  const bool diag = holds_diag(j, kb);
  const int dq = j & 3;
#pragma unroll
  for (int p = 0; p < WT; ++p) {
    const int64_t tr = t0 + 16 * (tg * WT + p);
#pragma unroll
    for (int q = 0; q < WE; ++q) {
      const int e = 16 * (eg * WE + q) + j;
      if (e < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t t = tr + 4 * kb + i;
          if (t < T) part[((int64_t)s * T + t) * E + e] = accD[p][q][i];
        }
      }
    }
    if (xnorm && diag && tr + j < T) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (dq == i) xsq[(int64_t)s * T + tr + j] = xsqD[p][i];
    }
  }
  if (wnorm && diag) {
#pragma unroll
    for (int q = 0; q < WE; ++q) {
      const int e = 16 * (eg * WE + q) + j;
      if (e < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (dq == i) wsq[(int64_t)s * E + e] = wsqD[q][i];
      }
    }
  }
}

// LDS of route_pick: the screen layout for kPickTT tokens, no ring and no
// K-split partials.
// Four waves, one token each (measured faster than 8 waves: Mixtral-shaped
// 57 -> 41 us for both kernels together).  With batches of at most 2 exact
// logits the kernel needs 86 VGPRs (five workgroups per CU); with one batch
// of up to 8 and one chunk round in flight, 116 (four per CU, still every
// token of a 4096-token batch in flight at once).
constexpr int kPickWaves = 4;
constexpr int kPickTT = kPickWaves;  // one token per wave
constexpr int kPickThreads = 64 * kPickWaves;
constexpr int kPickMaxE = 256;  // experts of the split screen
constexpr int kPartMaxSK = 8;   // most K splits of the split screen
__host__ __device__ constexpr ScreenLds pick_lds(int E) {
  ScreenLds o{};
  o.lg = 0;
  o.wn = o.lg + (int64_t)kPickTT * E * 8;
  o.xn = o.wn + ((int64_t)E * 4 + 15) / 16 * 16;
  o.xp = o.xn + kScreenTT * 4;
  o.sl = o.xp;  // no partials
  o.un = o.sl + (int64_t)kPickWaves * sizeof(SelSlots);
  o.total = o.un + ((int64_t)kPickWaves * E * 2 + 15) / 16 * 16;
  return o;
}

// Steps 2-4 from the partials: one workgroup of 8 waves per 8 tokens adds
// the splits (split order), the bias and the norms, then selects as
// route_staged does.
// CB: largest batch of exact logits, PRE: chunk rounds of their loads in
// flight (E = 256: one batch of 8 with one round, 95 us at the DeepSeek-V3
// shape against 111 us for batches of 2 with three rounds; E = 8: batches
// of 2, three rounds, at five workgroups per CU).
template <int M, int CB, int PRE>
__global__ __launch_bounds__(kPickThreads) void route_pick_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
    const double* __restrict__ part, const double* __restrict__ xsq,
    const double* __restrict__ wsq, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits_out, int64_t T, int64_t d, int E, int k, int SK) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const ScreenLds L = pick_lds(E);
  const ScreenSmem S(smem, L);
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kPickTT;
  // the splits' sums, each added in split order; every load of a thread is
  // issued before the first add (one memory latency instead of one per split)
  static_assert(kPickTT * kPickMaxE <= 4 * kPickThreads, "at most 4 logits per thread");
  static_assert(kPickMaxE <= kPickThreads, "one norm per thread");
  {
    double pw[kPartMaxSK], px[kPartMaxSK];
    const int64_t t_x = t0 + tid < T ? t0 + tid : T - 1;
#pragma unroll
    for (int sp = 0; sp < kPartMaxSK; ++sp) {
      pw[sp] = sp < SK && tid < E ? wsq[(int64_t)sp * E + tid] : 0.0;
      px[sp] = sp < SK && tid < kPickTT ? xsq[(int64_t)sp * T + t_x] : 0.0;
    }
    double qw = 0.0, qx = 0.0;
#pragma unroll
    for (int sp = 0; sp < kPartMaxSK; ++sp) {
      if (sp < SK) {
        qw += pw[sp];
        qx += px[sp];
      }
    }
    if (tid < E) S.wn[tid] = __double2float_ru(sqrt(qw));
    if (tid < kPickTT) S.xn[tid] = __double2float_ru(sqrt(qx));
  }
  {
    double pl[4][kPartMaxSK];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = tid + u * kPickThreads;
      const int tl = o / E, e = o % E;
      const int64_t t = t0 + tl < T ? t0 + tl : T - 1;
#pragma unroll
      for (int sp = 0; sp < kPartMaxSK; ++sp)
        pl[u][sp] = sp < SK && o < kPickTT * E ? part[((int64_t)sp * T + t) * E + e] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int o = tid + u * kPickThreads;
      if (o < kPickTT * E) {
        double v = 0.0;
#pragma unroll
        for (int sp = 0; sp < kPartMaxSK; ++sp)
          if (sp < SK) v += pl[u][sp];
        S.lg[o] = rank_value(v, bias, o % E);
      }
    }
  }
  __syncthreads();
  screen_select<M, kPickTT, CB, PRE>(S, x, Wr, bias, topk_idx, topk_w, logits_out, T, d, E, k, t0);
}

// Split count and scratch bytes of route_split for an NTB-token-block tile:
// the fewest splits (1, 2, 4 or 8) that give 256 workgroups, fewer if the
// scratch is smaller; 0 if not even one split fits.
struct SplitPlan {
  int SK, ntiles;
  size_t part_off, xsq_off, wsq_off, bytes;
};
inline bool plan_split(const Shape& s, int NTB, size_t scratch_bytes, SplitPlan* pl) {
  const int64_t ntiles = (s.T + 16 * NTB - 1) / (16 * NTB);
  const int64_t nsteps = (s.d + 63) / 64;
  int SK = 1;
  while (SK < kPartMaxSK && ntiles * SK < 256 && nsteps >= 2 * SK) SK *= 2;
  auto bytes = [&](int sk, size_t* a, size_t* b, size_t* c) {
    const size_t p = (size_t)sk * (size_t)s.T * (size_t)s.E * 8;
    const size_t xq = (size_t)sk * (size_t)s.T * 8;
    const size_t wq = (size_t)sk * (size_t)s.E * 8;
    *a = 0;
    *b = (p + 255) & ~(size_t)255;
    *c = *b + ((xq + 255) & ~(size_t)255);
    return *c + wq;
  };
  for (; SK >= 1; SK /= 2) {
    size_t a, b, c;
    const size_t total = bytes(SK, &a, &b, &c);
    if (total <= scratch_bytes) {
      *pl = SplitPlan{SK, (int)ntiles, a, b, c, total};
      return true;
    }
  }
  return false;
}

template <int NTB, int NEB, int WT, int WE, int M, int CB = 2, int PRE = kExactPre>
hipError_t launch_split(const Shape& s, const void* x, const void* Wr, const float* bias,
                        int32_t* idx, float* w, float* lo, const SplitPlan& pl,
                        unsigned char* scratch, hipStream_t st) {
  double* part = (double*)(scratch + pl.part_off);
  double* xq = (double*)(scratch + pl.xsq_off);
  double* wq = (double*)(scratch + pl.wsq_off);
  const unsigned grid1 = (unsigned)((((int64_t)pl.ntiles * pl.SK + 7) / 8) * 8);
  hipLaunchKernelGGL((route_part_kernel<NTB, NEB, WT, WE>), dim3(grid1), dim3(kScreenThreads), 0,
                     st, (const bf16_t*)x, (const bf16_t*)Wr, part, xq, wq, s.T, s.d, (int)s.E,
                     pl.SK, pl.ntiles);
  const unsigned grid2 = (unsigned)((s.T + kPickTT - 1) / kPickTT);
  hipLaunchKernelGGL((route_pick_kernel<M, CB, PRE>), dim3(grid2), dim3(kPickThreads),
                     (size_t)pick_lds((int)s.E).total, st, (const bf16_t*)x, (const bf16_t*)Wr,
                     bias, (const double*)part, (const double*)xq, (const double*)wq, idx, w, lo,
                     s.T, s.d, (int)s.E, (int)s.k, pl.SK);
  return hipGetLastError();
}

// route_split if it applies (bf16, 64 < T, E <= 256, the scratch holds the
// partials of at least one split) and pays: route_staged copies 128 expert
// rows per K step even for fewer experts, and streams all of W once per 16
// tokens, while route_split reads x twice and sums partials.  Measured:
// E = 8 (Mixtral shape) 82 -> 41 us, W of 3.7 MB (DeepSeek shape, E = 256)
// 127 -> 109 us, but E = 128 with W of 0.5 MB (fine-grained Zipf) 38.5 ->
// 44 us: route_split is taken for E <= 64 or W of at least 2 MB.  Else
// hipErrorNotSupported and nothing is launched.
inline bool split_applies(const Shape& s) {
  if (s.dt != MOE_DT_BF16 || s.T <= 64 || s.E > 256 || s.E * s.d * 2 >= ((int64_t)1 << 31))
    return false;
  return s.E <= 64 || s.E * s.d * 2 >= ((int64_t)2 << 20);
}
inline int split_ntb(const Shape& s) { return s.E <= 32 ? 8 : 4; }

hipError_t try_split(const Shape& s, const void* x, const void* Wr, const float* bias,
                     int32_t* idx, float* w, float* lo, void* scratch, size_t scratch_bytes,
                     hipStream_t st) {
  if (!scratch || !split_applies(s)) return hipErrorNotSupported;
  SplitPlan pl;
  unsigned char* sc = (unsigned char*)scratch;
  if (!plan_split(s, split_ntb(s), scratch_bytes, &pl)) return hipErrorNotSupported;
  if (s.E <= 16) return launch_split<8, 1, 1, 1, 1>(s, x, Wr, bias, idx, w, lo, pl, sc, st);
  if (s.E <= 32) return launch_split<8, 2, 2, 1, 1>(s, x, Wr, bias, idx, w, lo, pl, sc, st);
  if (s.E <= 64) return launch_split<4, 4, 2, 1, 1>(s, x, Wr, bias, idx, w, lo, pl, sc, st);
  if (s.E <= 128) return launch_split<4, 8, 2, 2, 2, 8, 1>(s, x, Wr, bias, idx, w, lo, pl, sc, st);
  return launch_split<4, 16, 2, 4, 4, 8, 1>(s, x, Wr, bias, idx, w, lo, pl, sc, st);
}

template <typename In>
hipError_t launch_small(const Shape& s, const void* x, const void* Wr, const float* bias,
                        int32_t* idx, float* w, float* lo, hipStream_t st) {
  // split each router row over KS lanes so that the E rows fill the block
  int KS = 1;
  while (KS < 64 && (int64_t)(kSmallThreads / (KS * 2)) >= s.E) KS *= 2;
  hipLaunchKernelGGL((route_small_kernel<In>), dim3((unsigned)s.T), dim3(kSmallThreads), 0, st,
                     (const In*)x, (const In*)Wr, bias, idx, w, lo, s.d, (int)s.E, (int)s.k, KS);
  return hipGetLastError();
}

template <typename In, int TT>
hipError_t launch_tiled(const Shape& s, const void* x, const void* Wr, const float* bias,
                        int32_t* idx, float* w, float* lo, hipStream_t st) {
  int P = 1;
  while (P < s.E && P < kMaxP) P <<= 1;
  if (P < 32) P = 32;  // keep the chunk split at most 8 ways
  const unsigned grid = (unsigned)((s.T + TT - 1) / TT);
  hipLaunchKernelGGL((route_tiled_kernel<In, TT>), dim3(grid), dim3(kThreads), 0, st,
                     (const In*)x, (const In*)Wr, bias, idx, w, lo, s.T, s.d, (int)s.E,
                     (int)s.k, P);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_dt(const Shape& s, const void* x, const void* Wr, const float* bias,
                     int32_t* idx, float* w, float* lo, hipStream_t st) {
  if (s.T <= 64) return launch_small<In>(s, x, Wr, bias, idx, w, lo, st);
  if constexpr (sizeof(In) == 2) {
    // allow more than 64 KB of dynamic LDS, once per device (the attribute
    // belongs to the device's copy of the kernel)
    static std::atomic<bool> lds_opt_in[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    const unsigned grid = (unsigned)((s.T + kScreenTT - 1) / kScreenTT);
    if (!lds_opt_in[dev].load(std::memory_order_acquire)) {
      // each kernel's largest dynamic LDS (its static rings come on top)
      const struct {
        const void* f;
        int64_t bytes;
      } opt[] = {{(const void*)route_staged_kernel<1>, screen_lds(128, true).total},
                 {(const void*)route_staged_kernel<2>, screen_lds(kStagedMaxE, false).total},
                 {(const void*)route_direct_kernel<2>, screen_lds(kMaxE, true).total}};
      for (const auto& o : opt) {
        e = hipFuncSetAttribute(o.f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)o.bytes);
        if (e != hipSuccess) return e;
      }
      lds_opt_in[dev].store(true, std::memory_order_release);
    }
    // up to 256 experts: operands staged through LDS, one block of 16
    // experts per wave up to 128 experts, two beyond; more experts: direct
    if (s.E <= 128) {
      const size_t lds = (size_t)screen_lds((int)s.E, true).total;
      hipLaunchKernelGGL(route_staged_kernel<1>, dim3(grid), dim3(kScreenThreads), lds, st,
                         (const bf16_t*)x, (const bf16_t*)Wr, bias, idx, w, lo, s.T, s.d,
                         (int)s.E, (int)s.k);
    } else if (s.E <= kStagedMaxE) {
      const size_t lds = (size_t)screen_lds((int)s.E, false).total;
      hipLaunchKernelGGL(route_staged_kernel<2>, dim3(grid), dim3(kScreenThreads), lds, st,
                         (const bf16_t*)x, (const bf16_t*)Wr, bias, idx, w, lo, s.T, s.d,
                         (int)s.E, (int)s.k);
    } else {
      const size_t lds = (size_t)screen_lds((int)s.E, true).total;
      hipLaunchKernelGGL(route_direct_kernel<2>, dim3(grid), dim3(kScreenThreads), lds, st,
                         (const bf16_t*)x, (const bf16_t*)Wr, bias, idx, w, lo, s.T, s.d,
                         (int)s.E, (int)s.k);
    }
    return hipGetLastError();
  } else {
    if (s.E > 512) return launch_tiled<In, 8>(s, x, Wr, bias, idx, w, lo, st);
    return launch_tiled<In, 16>(s, x, Wr, bias, idx, w, lo, st);
  }
}

}  // namespace

size_t route_workspace_bytes(const Shape& s) {
  SplitPlan pl;
  if (!split_applies(s) || !plan_split(s, split_ntb(s), ~(size_t)0, &pl)) return 0;
  return pl.bytes;
}

hipError_t launch_route(const Shape& s, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w,
                        float* logits_out, hipStream_t st, void* scratch,
                        size_t scratch_bytes) {
  if (s.T == 0) return hipSuccess;
  const hipError_t e =
      try_split(s, x, W_router, bias, topk_idx, topk_w, logits_out, scratch, scratch_bytes, st);
  if (e != hipErrorNotSupported) return e;
  if (s.dt == MOE_DT_BF16)
    return launch_dt<bf16_t>(s, x, W_router, bias, topk_idx, topk_w, logits_out, st);
  return launch_dt<float>(s, x, W_router, bias, topk_idx, topk_w, logits_out, st);
}

}  // namespace moe
