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
// Three logit layouts, one top-k:
//   route_small (T <= 64, decode): one workgroup per token; thread (e, ks)
//     sums the 16-byte chunks ks, ks+KS, ... of router row e against the
//     token row straight from global memory (coalesced across the KS lanes of
//     an expert), then the KS partials are combined by a fixed butterfly.
//   route_screen (bf16, large T): bf16 MFMA screen with a rigorous error
//     bound, fp64 logits only for the experts that can still be selected.
//   route_tiled (fp32, large T): one workgroup per TT tokens; x and W chunks
//     are staged through LDS and thread (ks, e) keeps TT running logits, so
//     each router row is read once per TT tokens.
//   topk_wave: one wave per token; each lane holds ceil(E/64) logits and k
//     rounds of a wave-wide argmax (butterfly over (value, index)) pick the
//     experts.
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

// Top-k of one token's logits (LDS row of E values) by one wave; writes the
// k expert ids in rank order and their renormalised weights.  k <= 64.
// Lane l owns experts l, l+64, ...; each round every lane rescans its
// unpicked logits from LDS and a butterfly over (value, index) finds the
// wave-wide best.
__device__ void topk_wave(const double* logits, const float* __restrict__ bias, int E,
                          int k, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  uint32_t taken = 0;
  double sel_v0 = 0.0, wsum = 0.0;
  double my_ex = 0.0;  // lane j keeps exp(l_j - l_0)
  int my_e = 0;
  for (int j = 0; j < k; ++j) {
    double bv = -INFINITY;
    int be = 0x7fffffff;
    for (int m = 0, e = lane; e < E; ++m, e += 64) {
      if ((taken >> m) & 1u) continue;
      double v = logits[e];
      if (bias) v += (double)bias[e];
      if (v != v) v = -INFINITY;  // NaN ranks last
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
    if (j == 0) sel_v0 = bv;
    const double ex = exp(bv - sel_v0);
    wsum += ex;
    if (lane == j) {
      my_ex = ex;
      my_e = be;
    }
  }
  if (lane < k) {
    idx_out[lane] = my_e;
    w_out[lane] = (float)(my_ex / wsum);
  }
}

// ------------------------------------------------------------ route_small
constexpr int kSmallThreads = 1024;


template <typename In>
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(
    const In* __restrict__ x, const In* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t d, int E, int k,
    int KS) {
  __shared__ double logits[kMaxE];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int per_pass = kSmallThreads / KS;
  const int ks = tid % KS;
  const int64_t nchunk = d / 8;
  const In* xr = x + t * d;
  // 8-element chunks of x and W in flight per thread (128 bytes of each)
  constexpr int kSmallBatch = sizeof(In) == 2 ? 8 : 4;
  for (int e0 = 0; e0 < E; e0 += per_pass) {
    const int e = e0 + tid / KS;
    double acc = 0.0;
    if (e < E) {
      const In* wr = Wr + (int64_t)e * d;
      // chunks ks, ks+KS, ... in order, kSmallBatch of them loaded at once
      // (chunks past the row read chunk 0 and are not used)
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
    if (ks == 0 && e < E) logits[e] = acc;
  }
  __syncthreads();
  if (tid < 64) topk_wave(logits, bias, E, k, topk_idx + t * k, topk_w + t * k);
}

// ------------------------------------------------------------ route_tiled
template <int TT>
struct TiledSmem {
  static constexpr int kE = (TT == 16) ? 512 : 1024;
  double logits[TT][kE];         // 64 KB
  float w[kKC][kMaxP];           // staged router weights, transposed (32 KB)
  double xs[TT][kKC];            // staged token chunk (fp64)
  double part[kThreads][TT];     // k-split partial sums (32 KB at TT=16)
};

template <typename In, int TT>
__global__ __launch_bounds__(kThreads) void route_tiled_kernel(
    const In* __restrict__ x, const In* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t T, int64_t d,
    int E, int k, int P) {
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
        sm.logits[t][e0 + e_loc] = s;
      }
    }
    __syncthreads();
  }

  const int wave = tid >> 6;
  for (int t = wave; t < TT; t += kThreads / 64) {
    if (t0 + t >= T) break;
    topk_wave(sm.logits[t], bias, E, k, topk_idx + (t0 + t) * k, topk_w + (t0 + t) * k);
  }
}

// ----------------------------------------------------------- route_screen
// bf16, large T.  Exact fp64 logits of every (token, expert) pair cost
// 2*T*E*d fp64 flops; instead the experts are screened with bf16 MFMA and
// only the few that can still be in a token's top-k get an fp64 logit:
//   1. MFMA screen: L~[t,e] = sum over K chunks of 32 of the chunk's MFMA
//      result (fp32, started from zero), the chunk sums added in fp64.
//      Every bf16 product is exact in fp32, so the only error is the
//      rounding inside each 32-term chunk sum: |L~ - L| <= b[t,e] with
//      b = kScreenRel * ||x_t|| * ||w_e||  (Cauchy-Schwarz bounds the sum of
//      |products|; kScreenRel = 2^-17 covers 32 roundings of 2^-23 each with
//      a factor of two to spare, plus the fp32 norms' own rounding).
//   2. With lo = L~ - b, hi = L~ + b and tau = the k-th largest lo, an
//      expert whose hi < tau is below k others for certain; the rest are
//      the candidates (k of them, rarely a few more).
//   3. Candidates get their fp64 logit (same fixed summation order for every
//      expert, so identical rows still tie exactly); the top-k and weights
//      are taken over these exact logits by topk_wave.
// The result is the same selection and weights as the fp64-everywhere path.
constexpr int kScreenTT = 16;                  // token rows of the screen (LDS rows)
constexpr double kScreenRel = 7.62939453125e-06;  // 2^-17
constexpr int kCandBatch = 4;                  // candidates per fp64 pass

// LDS layout of route_screen (bytes), sized by E at launch:
//   lg    [16][E] double   screen logits, then exact logits / -inf
//   wsq   [E]     float    ||w_e||^2
//   xsq   [16]    float    ||x_t||^2
//   union { part [16 items][16][16] double (screen K-split partials, E < 256),
//           cand [4 waves][E] int      (candidate lists) }
struct ScreenLds {
  int64_t lg, wsq, xsq, un, total;
};
__host__ __device__ inline ScreenLds screen_lds(int E) {
  ScreenLds o;
  o.lg = 0;
  o.wsq = o.lg + (int64_t)kScreenTT * E * 8;
  o.xsq = o.wsq + ((int64_t)E * 4 + 15) / 16 * 16;
  o.un = o.xsq + kScreenTT * 4;
  const int64_t part = E < 256 ? 16 * 16 * 16 * 8 : 0;
  const int64_t cand = (int64_t)(kThreads / 64) * E * 4;
  o.total = o.un + (part > cand ? part : cand);
  return o;
}

__global__ __launch_bounds__(kThreads, 2) void route_screen_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t T, int64_t d, int E,
    int k, int tok) {
  // tok (8 or 16): tokens per workgroup; screen rows past them repeat the last
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const ScreenLds L = screen_lds(E);
  double* lg = reinterpret_cast<double*>(smem + L.lg);  // [16][E]
  float* wsq_s = reinterpret_cast<float*>(smem + L.wsq);
  float* xsq_s = reinterpret_cast<float*>(smem + L.xsq);
  double* part = reinterpret_cast<double*>(smem + L.un);  // [16][16][16]
  int* cand = reinterpret_cast<int*>(smem + L.un);        // [4][E]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 15, kb = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * tok;
  const int jt = j < tok ? j : tok - 1;
  const int64_t tj = t0 + jt < T ? t0 + jt : T - 1;  // padding tokens repeat the last
  const bf16_t* xa = x + tj * d;
  const int64_t nch = (d + 31) / 32;               // K chunks of 32

  // ---- 1. MFMA screen.  A pass covers up to 16 blocks of 16 experts; with
  // fewer blocks (small E) K is split KS ways too.  The pass's
  // (block, K-split) items are dealt 4 per wave; item i = q*4 + wave.
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int nbp = min(16, (E - e0 + 15) / 16);
    int KS = 1;  // K splits only in the single pass of E < 256 (LDS holds part then)
    if (E < 256)
      while (nbp * KS * 2 <= 16) KS *= 2;
    const bf16_t* wb[4];
    int ks_of[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int item = q * 4 + wave;
      live[q] = item < nbp * KS;
      const int nb = live[q] ? item % nbp : 0;
      ks_of[q] = live[q] ? item / nbp : 0;
      const int e = e0 + 16 * nb + j;
      wb[q] = Wr + (int64_t)(e < E ? e : E - 1) * d;
    }
    double acc[4][4];
    float wsq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][i] = 0.0;
    // loads of K step `it` (clamped past K, zeroed at use), two register sets
    // alternating so one step's loads are in flight while the other computes
    auto ld = [&](int64_t it, u32x4 (&a)[4], u32x4 (&b)[4], bool (&ok)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t kk = (it * KS + ks_of[q]) * 32 + 8 * kb;
        ok[q] = live[q] && kk < d;
        const int64_t ka = ok[q] ? kk : 0;
        a[q] = ldg16(xa + ka);
        b[q] = ldg16(wb[q] + ka);
      }
    };
    auto mm = [&](const u32x4 (&a)[4], const u32x4 (&b)[4], const bool (&ok)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 aa = zero_unless(ok[q], a[q]);
        const u32x4 bb = zero_unless(ok[q], b[q]);
        const uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          wsq[q] = fmaf(bf16lo(bw[h]), bf16lo(bw[h]), wsq[q]);
          wsq[q] = fmaf(bf16hi(bw[h]), bf16hi(bw[h]), wsq[q]);
        }
        const f32x4 r = mfma16(aa, bb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[q][i] += (double)r[i];
      }
    };
    const int64_t nit = (nch + KS - 1) / KS;
    u32x4 a0[4], b0[4], a1[4], b1[4];
    bool o0[4], o1[4];
    ld(0, a0, b0, o0);
    int64_t it = 0;
    for (; it + 2 <= nit; it += 2) {
      ld(it + 1, a1, b1, o1);
      mm(a0, b0, o0);
      ld(it + 2, a0, b0, o0);
      mm(a1, b1, o1);
    }
    if (it < nit) mm(a0, b0, o0);
    // partial results: lane holds token 4*kb + i, expert 16*nb + j
    if (KS == 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + 16 * (q * 4 + wave) + j;
        if (live[q] && e < E) {
#pragma unroll
          for (int i = 0; i < 4; ++i) lg[(4 * kb + i) * E + e] = acc[q][i];
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (live[q]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) part[((q * 4 + wave) * 16 + 4 * kb + i) * 16 + j] = acc[q][i];
        }
      }
    }
    // ||w||^2 of each K-split, summed over the 4 lanes of a column
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float sq = wsq[q] + __shfl_xor(wsq[q], 16, 64);
      sq += __shfl_xor(sq, 32, 64);
      wsq[q] = sq;
    }
    __syncthreads();
    if (KS > 1) {
      // add the K-split partials in split order; items nb + nbp*ks
      for (int o = tid; o < nbp * 256; o += kThreads) {
        const int nb = o / 256, r = (o / 16) % 16, c = o % 16;
        const int e = e0 + 16 * nb + c;
        double sacc = 0.0;
        for (int ks = 0; ks < KS; ++ks) sacc += part[((nb + nbp * ks) * 16 + r) * 16 + c];
        if (e < E) lg[r * E + e] = sacc;
      }
    }
    // ||w_e||^2: the split partials, again in split order (through LDS)
    __syncthreads();
    float* wpart = reinterpret_cast<float*>(part);  // [16 items][16]
    if (kb == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (live[q]) wpart[(q * 4 + wave) * 16 + j] = wsq[q];
    }
    __syncthreads();
    if (tid < nbp * 16) {
      const int nb = tid / 16, c = tid % 16;
      float sq = 0.f;
      for (int ks = 0; ks < KS; ++ks) sq += wpart[(nb + nbp * ks) * 16 + c];
      if (e0 + tid < E) wsq_s[e0 + tid] = sq;
    }
    __syncthreads();
  }
  // ||x_t||^2 (wave 0: lane (j, kb) sums 16-byte chunks kb, kb+4, ... of
  // token j, eight loads in flight, then across kb)
  if (wave == 0) {
    float xsq = 0.f;
    const int64_t n8 = d / 8;
    for (int64_t c0 = kb; c0 < n8; c0 += 32) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t c = c0 + 4 * u;
        v[u] = zero_unless(c < n8, ldg16(xa + (c < n8 ? c : 0) * 8));
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t aw[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          xsq = fmaf(bf16lo(aw[h]), bf16lo(aw[h]), xsq);
          xsq = fmaf(bf16hi(aw[h]), bf16hi(aw[h]), xsq);
        }
      }
    }
    xsq += __shfl_xor(xsq, 16, 64);
    xsq += __shfl_xor(xsq, 32, 64);
    if (kb == 0) xsq_s[j] = xsq;
  }
  __syncthreads();

  // ---- 2./3. one wave per token
  int* mycand = cand + wave * E;
  for (int tl = wave; tl < tok; tl += kThreads / 64) {
    const int64_t t = t0 + tl;
    if (t >= T) break;
    double* row = lg + (int64_t)tl * E;
    // fp32 norms carry relative error <= d * 2^-24; the factor 1.001 covers it
    const double xn = sqrt((double)xsq_s[tl]) * 1.001;
    auto bound = [&](int e) { return kScreenRel * xn * sqrt((double)wsq_s[e]) + 1e-30; };
    // tau = k-th largest lower bound (ties broken by index, as everywhere)
    uint32_t taken = 0;
    double tau = 0.0;
    for (int jj = 0; jj < k; ++jj) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
      for (int m = 0, e = lane; e < E; ++m, e += 64) {
        if ((taken >> m) & 1u) continue;
        double lo = row[e] + (bias ? (double)bias[e] : 0.0) - bound(e);
        if (lo != lo) lo = -INFINITY;
        if (better(lo, e, bv, be)) {
          bv = lo;
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
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      tau = bv;
    }
    // candidates: hi >= tau, compacted in expert order
    int ncand = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      bool c = false;
      if (e < E) {
        const double hi = row[e] + (bias ? (double)bias[e] : 0.0) + bound(e);
        c = !(hi < tau);
      }
      const uint64_t m = __ballot(c);
      if (c) mycand[ncand + __popcll(m & ((1ull << lane) - 1ull))] = e;
      ncand += __popcll(m);
    }
    // every non-candidate drops out of the top-k
    for (int e = lane; e < E; e += 64) row[e] = -INFINITY;
    // fp64 logits of the candidates: lane l sums 16-byte chunks l, l+64, ...
    const bf16_t* xt = x + t * d;
    const int64_t n8 = d / 8;
    for (int c0 = 0; c0 < ncand; c0 += kCandBatch) {
      double acc[kCandBatch];
      const bf16_t* wr[kCandBatch];
#pragma unroll
      for (int u = 0; u < kCandBatch; ++u) {
        acc[u] = 0.0;
        const int ci = c0 + u < ncand ? c0 + u : ncand - 1;
        wr[u] = Wr + (int64_t)mycand[ci] * d;
      }
      for (int64_t ch = lane; ch < n8; ch += 128) {
        // two chunks per iteration: ch and ch + 64 (if inside the row)
        const bool two = ch + 64 < n8;
        const int64_t ch2 = two ? ch + 64 : ch;
        const u32x4 xv0 = ldg16(xt + ch * 8), xv1 = ldg16(xt + ch2 * 8);
        u32x4 wv0[kCandBatch], wv1[kCandBatch];
#pragma unroll
        for (int u = 0; u < kCandBatch; ++u) {
          wv0[u] = ldg16(wr[u] + ch * 8);
          wv1[u] = ldg16(wr[u] + ch2 * 8);
        }
        const uint32_t x0[4] = {xv0.x, xv0.y, xv0.z, xv0.w};
        const uint32_t x1[4] = {xv1.x, xv1.y, xv1.z, xv1.w};
#pragma unroll
        for (int u = 0; u < kCandBatch; ++u) {
          const uint32_t w0[4] = {wv0[u].x, wv0[u].y, wv0[u].z, wv0[u].w};
          const uint32_t w1[4] = {wv1[u].x, wv1[u].y, wv1[u].z, wv1[u].w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            acc[u] = fma((double)bf16lo(x0[h]), (double)bf16lo(w0[h]), acc[u]);
            acc[u] = fma((double)bf16hi(x0[h]), (double)bf16hi(w0[h]), acc[u]);
          }
          if (two) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
              acc[u] = fma((double)bf16lo(x1[h]), (double)bf16lo(w1[h]), acc[u]);
              acc[u] = fma((double)bf16hi(x1[h]), (double)bf16hi(w1[h]), acc[u]);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCandBatch; ++u) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) acc[u] += __shfl_xor(acc[u], off, 64);
      }
      if (lane == 0) {
#pragma unroll
        for (int u = 0; u < kCandBatch; ++u)
          if (c0 + u < ncand) row[mycand[c0 + u]] = acc[u];
      }
    }
    topk_wave(row, bias, E, k, topk_idx + t * k, topk_w + t * k);
  }
}

template <typename In>
hipError_t launch_small(const Shape& s, const void* x, const void* Wr, const float* bias,
                        int32_t* idx, float* w, hipStream_t st) {
  // split each router row over KS lanes so that the E rows fill the block
  int KS = 1;
  while (KS < 64 && (int64_t)(kSmallThreads / (KS * 2)) >= s.E) KS *= 2;
  hipLaunchKernelGGL((route_small_kernel<In>), dim3((unsigned)s.T), dim3(kSmallThreads), 0, st,
                     (const In*)x, (const In*)Wr, bias, idx, w, s.d, (int)s.E, (int)s.k, KS);
  return hipGetLastError();
}

template <typename In, int TT>
hipError_t launch_tiled(const Shape& s, const void* x, const void* Wr, const float* bias,
                        int32_t* idx, float* w, hipStream_t st) {
  int P = 1;
  while (P < s.E && P < kMaxP) P <<= 1;
  if (P < 32) P = 32;  // keep the chunk split at most 8 ways
  const unsigned grid = (unsigned)((s.T + TT - 1) / TT);
  hipLaunchKernelGGL((route_tiled_kernel<In, TT>), dim3(grid), dim3(kThreads), 0, st,
                     (const In*)x, (const In*)Wr, bias, idx, w, s.T, s.d, (int)s.E,
                     (int)s.k, P);
  return hipGetLastError();
}

template <typename In>
hipError_t launch_dt(const Shape& s, const void* x, const void* Wr, const float* bias,
                     int32_t* idx, float* w, hipStream_t st) {
  if (s.T <= 64) return launch_small<In>(s, x, Wr, bias, idx, w, st);
  if constexpr (sizeof(In) == 2) {
    const size_t lds = (size_t)screen_lds((int)s.E).total;
    // allow more than 64 KB of dynamic LDS, once per device (the attribute
    // belongs to the device's copy of the kernel)
    static std::atomic<bool> lds_opt_in[kMaxDevices];
    static std::atomic<int> cu_count[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int cus = cu_count[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    // 16 tokens per workgroup; 8 when that still leaves workgroup slots (two
    // per CU) empty and the router matrix is small enough (<= 1 MB) for the
    // extra workgroups to re-read it cheaply (measured: E=128, d=2048 faster;
    // E=256, d=7168 and T=8192 slower)
    int tok = kScreenTT;
    if ((s.T + kScreenTT - 1) / kScreenTT < 2 * (int64_t)cus && s.E * s.d * 2 <= (1 << 20))
      tok = 8;
    const unsigned grid = (unsigned)((s.T + tok - 1) / tok);
    if (!lds_opt_in[dev].load(std::memory_order_acquire)) {
      e = hipFuncSetAttribute((const void*)route_screen_kernel,
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)screen_lds(1024).total);
      if (e != hipSuccess) return e;
      lds_opt_in[dev].store(true, std::memory_order_release);
    }
    hipLaunchKernelGGL(route_screen_kernel, dim3(grid), dim3(kThreads), lds, st,
                       (const bf16_t*)x, (const bf16_t*)Wr, bias, idx, w, s.T, s.d, (int)s.E,
                       (int)s.k, tok);
    return hipGetLastError();
  } else {
    if (s.E > 512) return launch_tiled<In, 8>(s, x, Wr, bias, idx, w, st);
    return launch_tiled<In, 16>(s, x, Wr, bias, idx, w, st);
  }
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w,
                        hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.dt == MOE_DT_BF16)
    return launch_dt<bf16_t>(s, x, W_router, bias, topk_idx, topk_w, st);
  return launch_dt<float>(s, x, W_router, bias, topk_idx, topk_w, st);
}

}  // namespace moe
