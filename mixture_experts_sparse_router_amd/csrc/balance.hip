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
// balance_partial: one wave per token (8 tokens per wave, 4 waves); lane l
//   owns experts l, l+64, ...: wave max, exp(L - max) in fp32, their sum in
//   fp64 by a fixed butterfly, p = exp / sum; each lane adds its experts' p
//   over the wave's tokens in fp64, and the 4 waves are added in wave order
//   into partial[block][E].
// balance_final: one workgroup; thread e adds partial[b][e] in block order
//   and divides by T; the E loss terms are added by a fixed tree.
// Every sum has a fixed order, so repeated calls are bitwise identical.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kBalWaves = 4;
constexpr int kBalTokensPerWave = 8;
constexpr int kBalTokens = kBalWaves * kBalTokensPerWave;  // tokens per workgroup
constexpr int kBalMaxM = 16;                              // experts per lane (E <= 1024)
constexpr int kBalMaxE = 64 * kBalMaxM;
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(64 * kBalWaves) void balance_partial_kernel(
    const float* __restrict__ logits, double* __restrict__ partial, int64_t T, int E) {
  __shared__ double part[kBalWaves][kBalMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double acc[kBalMaxM];
#pragma unroll
  for (int q = 0; q < kBalMaxM; ++q) acc[q] = 0.0;
  const int64_t t0 = (int64_t)blockIdx.x * kBalTokens + (int64_t)wave * kBalTokensPerWave;
  for (int i = 0; i < kBalTokensPerWave; ++i) {
    const int64_t t = t0 + i;
    if (t >= T) break;
    const float* row = logits + t * E;
    float v[kBalMaxM];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kBalMaxM; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? row[e] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    double z = 0.0;
#pragma unroll
    for (int q = 0; q < kBalMaxM; ++q) {
      v[q] = lane + 64 * q < E ? expf(v[q] - m) : 0.f;
      z += (double)v[q];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
    const double rz = 1.0 / z;
#pragma unroll
    for (int q = 0; q < kBalMaxM; ++q) acc[q] += (double)v[q] * rz;
  }
#pragma unroll
  for (int q = 0; q < kBalMaxM; ++q) {
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
  __shared__ double terms[kFinalThreads];
  const int e = threadIdx.x;
  const double u = 1.0 / (double)E;
  double term = 0.0;
  if (e < E) {
    double s = 0.0;
    for (int b = 0; b < nblocks; ++b) s += partial[(int64_t)b * E + e];
    const double imp = s / (double)T;  // no tokens: 0 / 0
    importance[e] = imp;
    term = u * (log(u) - log(imp + 1e-8));
  }
  terms[e] = term;
  __syncthreads();
  for (int h = kFinalThreads / 2; h >= 1; h >>= 1) {
    if (e < h) terms[e] += terms[e + h];
    __syncthreads();
  }
  if (e == 0) *loss = terms[0] / (double)E;
}

}  // namespace

int64_t balance_partials(int64_t T) { return (T + kBalTokens - 1) / kBalTokens; }

hipError_t launch_balance(const Shape& s, const float* logits, double* partial,
                          double* importance, double* loss, hipStream_t st) {
  const int64_t nb = balance_partials(s.T);
  if (nb > 0)
    hipLaunchKernelGGL(balance_partial_kernel, dim3((unsigned)nb), dim3(64 * kBalWaves), 0, st,
                       logits, partial, s.T, (int)s.E);
  hipLaunchKernelGGL(balance_final_kernel, dim3(1), dim3(kFinalThreads), 0, st, partial,
                     (int)nb, s.T, (int)s.E, importance, loss);
  return hipGetLastError();
}

}  // namespace moe
