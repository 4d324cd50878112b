// balance.hip -- load statistics of the router: each expert's importance
// (its softmax probability averaged over the tokens) and the balance loss.
//
// Balance loss (yunthe "分工的艺术" page, section 3.1, load balance loss):
// the gate averaged over the batch is compared with the uniform
// distribution u = 1/E by a KL divergence, reduced as a batch mean over the
// E-long vector:
//   loss = (1/E) sum_e u (log u - log(imp_e + 1e-8)),
//   imp_e = (1/T) sum_t softmax(L_t)_e,
// where the gate is the softmax over all experts (that page's section 1.1
// gating code) of the router logits L (bias included).
//
// Input: the logits [T, E] fp32 that the route kernels write when asked.
// balance_partial: 16 tokens per workgroup, 4 per wave; lane l owns experts
//   l, l+64, ... (M of them).  A wave loads its 4 tokens' logits at once,
//   then per token: wave max, exp(L - max) in fp32, their sum in fp64 by a
//   fixed butterfly, p = exp / sum; each lane adds its experts' p over the
//   wave's tokens in fp64, and the 4 waves are added in wave order into
//   partial[block][E].
// balance_final: one workgroup of 1024 threads; P = 1024 / E' threads per
//   expert (E' = E rounded up to a power of two, at least 64) add strided
//   slices of the partials with four running sums, the P slices are added in
//   slice order, imp = sum / T; the E loss terms are added by a fixed tree.
// Every sum has a fixed order, so repeated calls are bitwise identical.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kBalWaves = 4;
constexpr int kBalTokensPerWave = kBalTokens / kBalWaves;
constexpr int kBalMaxE = 1024;
constexpr int kFinalThreads = 1024;

template <int M>
__global__ __launch_bounds__(64 * kBalWaves) void balance_partial_kernel(
    const float* __restrict__ logits, double* __restrict__ partial, int64_t T, int E) {
  __shared__ double part[kBalWaves][kBalMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * kBalTokens + (int64_t)wave * kBalTokensPerWave;
  // every load issued before any use: rows past T and experts past E read
  // element 0 and are masked below
  float v[kBalTokensPerWave][M];
#pragma unroll
  for (int i = 0; i < kBalTokensPerWave; ++i) {
#pragma unroll
    for (int q = 0; q < M; ++q) {
      const int e = lane + 64 * q;
      const bool ok = t0 + i < T && e < E;
      v[i][q] = logits[ok ? (t0 + i) * E + e : 0];
    }
  }
  double acc[M];
#pragma unroll
  for (int q = 0; q < M; ++q) acc[q] = 0.0;
#pragma unroll
  for (int i = 0; i < kBalTokensPerWave; ++i) {
    if (t0 + i >= T) break;
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < M; ++q)
      if (lane + 64 * q < E) m = fmaxf(m, v[i][q]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    float ex[M];
    double z = 0.0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      ex[q] = lane + 64 * q < E ? expf(v[i][q] - m) : 0.f;
      z += (double)ex[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
    const double rz = 1.0 / z;
#pragma unroll
    for (int q = 0; q < M; ++q) acc[q] += (double)ex[q] * rz;
  }
#pragma unroll
  for (int q = 0; q < M; ++q) {
    const int e = lane + 64 * q;
    if (e < E) part[wave][e] = acc[q];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64 * kBalWaves) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kBalWaves; ++w) s += part[w][e];
    partial[(int64_t)blockIdx.x * E + e] = s;
  }
}

__global__ __launch_bounds__(kFinalThreads) void balance_final_kernel(
    const double* __restrict__ partial, int nblocks, int64_t T, int E,
    double* __restrict__ importance, double* __restrict__ loss) {
  __shared__ double red[kFinalThreads];
  const int tid = threadIdx.x;
  int Ep = 64;
  while (Ep < E) Ep <<= 1;
  const int P = kFinalThreads / Ep;  // threads per expert
  const int e = tid % Ep, slice = tid / Ep;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (e < E) {
    int b = slice;
    for (; b + 3 * P < nblocks; b += 4 * P) {
      a0 += partial[(int64_t)b * E + e];
      a1 += partial[(int64_t)(b + P) * E + e];
      a2 += partial[(int64_t)(b + 2 * P) * E + e];
      a3 += partial[(int64_t)(b + 3 * P) * E + e];
    }
    for (; b < nblocks; b += P) a0 += partial[(int64_t)b * E + e];
  }
  red[tid] = (a0 + a1) + (a2 + a3);
  __syncthreads();
  const double u = 1.0 / (double)E;
  double term = 0.0;
  if (slice == 0 && e < E) {
    double s = 0.0;
    for (int q = 0; q < P; ++q) s += red[q * Ep + e];
    const double imp = s / (double)T;  // no tokens: 0 / 0
    importance[e] = imp;
    term = u * (log(u) - log(imp + 1e-8));
  }
  __syncthreads();
  red[tid] = term;
  __syncthreads();
  for (int h = kFinalThreads / 2; h >= 1; h >>= 1) {
    if (tid < h) red[tid] += red[tid + h];
    __syncthreads();
  }
  if (tid == 0) *loss = red[0] / (double)E;
}

}  // namespace

hipError_t launch_balance(const Shape& s, const float* logits, double* partial,
                          double* importance, double* loss, hipStream_t st) {
  const int64_t nb = balance_partials(s.T);
  if (nb > 0) {
    const int E = (int)s.E;
#define MOE_BAL(m)                                                                        \
  hipLaunchKernelGGL(balance_partial_kernel<m>, dim3((unsigned)nb), dim3(64 * kBalWaves), 0, \
                     st, logits, partial, s.T, E)
    if (E <= 64) MOE_BAL(1);
    else if (E <= 128) MOE_BAL(2);
    else if (E <= 256) MOE_BAL(4);
    else MOE_BAL(16);
#undef MOE_BAL
  }
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, partial,
                     (int)nb, s.T, (int)s.E, importance, loss);
  return hipGetLastError();
}

}  // namespace moe
