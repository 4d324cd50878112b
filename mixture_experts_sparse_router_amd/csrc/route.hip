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
// Layout: one workgroup (256 threads, 4 waves) routes TT tokens.
//   Phase 1 -- logits.  Experts are taken in passes of P (a power of two,
//   P <= 256); thread (ks, e) accumulates the TT logits of expert e over the
//   k-slice ks of every staged K chunk, in fp64 (products of bf16 or fp32
//   inputs are exact in fp64).  x and W chunks are staged through LDS.  The
//   KS = 256/P partial sums are added in fixed order, so the result does not
//   depend on scheduling.  Logits stay in LDS.
//   Phase 2 -- one wave per token: each lane holds ceil(E/64) logits; k rounds
//   of a wave-wide argmax (butterfly over (value, index)) pick the experts.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKC = 32;          // K elements per staged chunk
constexpr int kMaxP = 256;       // experts per pass

template <int TT>
struct RouteSmem {
  static constexpr int kMaxE = (TT == 16) ? 512 : 1024;
  double logits[TT][kMaxE];      // 64 KB
  float w[kKC][kMaxP];           // staged router weights, transposed (32 KB)
  double xs[TT][kKC];            // staged token chunk (fp64)
  double part[kThreads][TT];     // k-split partial sums (32 KB at TT=16)
};

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

// (value, index) order of the ranking: larger value first, then lower index.
__device__ __forceinline__ bool better(double v, int e, double bv, int be) {
  return v > bv || (v == bv && e < be);
}

template <typename In, int TT>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const In* __restrict__ x, const In* __restrict__ Wr, const float* __restrict__ bias,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int64_t T, int64_t d,
    int E, int k, int P) {
  __shared__ RouteSmem<TT> sm;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int KS = kThreads / P;     // k-splits per chunk
  const int e_loc = tid % P;
  const int ks = tid / P;

  // ---------------- phase 1: logits
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

  // ---------------- phase 2: top-k per token, one wave per token
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int M = (E + 63) / 64;     // logits per lane (<= 16)
  for (int t = wave; t < TT; t += kThreads / 64) {
    if (t0 + t >= T) break;
    double v[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int e = lane + 64 * m;
      double val = -INFINITY;
      if (m < M && e < E) {
        val = sm.logits[t][e];
        if (bias) val += (double)bias[e];
        if (val != val) val = -INFINITY;  // NaN ranks last
      }
      v[m] = val;
    }
    uint32_t taken = 0;
    double sel_v0 = 0.0, wsum = 0.0;
    double my_ex = 0.0;              // lane j keeps exp(l_j - l_0)
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      double bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const int e = lane + 64 * m;
        if (m < M && e < E && !((taken >> m) & 1u) && better(v[m], e, bv, be)) {
          bv = v[m];
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
      topk_idx[(t0 + t) * k + lane] = my_e;
      topk_w[(t0 + t) * k + lane] = (float)(my_ex / wsum);
    }
  }
}

template <typename In, int TT>
hipError_t launch_t(const Shape& s, const void* x, const void* Wr, const float* bias,
                    int32_t* idx, float* w, hipStream_t st) {
  int P = 1;
  while (P < s.E && P < kMaxP) P <<= 1;
  if (P < 32) P = 32;  // keep the chunk split at most 8 ways
  const unsigned grid = (unsigned)((s.T + TT - 1) / TT);
  hipLaunchKernelGGL((route_kernel<In, TT>), dim3(grid), dim3(kThreads), 0, st,
                     (const In*)x, (const In*)Wr, bias, idx, w, s.T, s.d, (int)s.E,
                     (int)s.k, P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Shape& s, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w,
                        hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const bool big = s.E > 512;
  if (s.dt == MOE_DT_BF16)
    return big ? launch_t<bf16_t, 8>(s, x, W_router, bias, topk_idx, topk_w, st)
               : launch_t<bf16_t, 16>(s, x, W_router, bias, topk_idx, topk_w, st);
  return big ? launch_t<float, 8>(s, x, W_router, bias, topk_idx, topk_w, st)
             : launch_t<float, 16>(s, x, W_router, bias, topk_idx, topk_w, st);
}

}  // namespace moe
