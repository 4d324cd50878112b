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
// Two logit layouts, one top-k:
//   route_small (T <= 64, decode): one workgroup per token; thread (e, ks)
//     sums the 16-byte chunks ks, ks+KS, ... of router row e against the
//     token row straight from global memory (coalesced across the KS lanes of
//     an expert), then the KS partials are combined by a fixed butterfly.
//   route_tiled (large T): one workgroup per TT tokens; x and W chunks are
//     staged through LDS and thread (ks, e) keeps TT running logits, so each
//     router row is read once per TT tokens.
//   topk_wave: one wave per token; each lane holds ceil(E/64) logits and k
//     rounds of a wave-wide argmax (butterfly over (value, index)) pick the
//     experts.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKC = 32;          // K elements per staged chunk (tiled)
constexpr int kMaxP = 256;       // experts per pass (tiled)
constexpr int kMaxE = 1024;

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
  if (s.E > 512) return launch_tiled<In, 8>(s, x, Wr, bias, idx, w, st);
  return launch_tiled<In, 16>(s, x, Wr, bias, idx, w, st);
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
