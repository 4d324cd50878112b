// combine.hip -- weighted un-permute of the expert outputs back to token order.
//
// y[t] = sum_{j<k} w[t,j] * out[slot_pos[t*k+j]]  (+ every shared expert row)
// (copies with slot_pos < 0, dropped by the permutation, add nothing)
// The output is the routing-weighted sum of the selected experts' outputs
// only (Baidu "MoE稀疏架构是什么" page, section 四), gathered and reordered
// back to token order after the grouped GEMM (aitoday "MoEs in Transformers"
// page, section "Expert Backend").  Accumulation is fp32 in the fixed order
// j = 0..k-1 then the shared experts: no atomics, bitwise reproducible.
//
// One workgroup per token row; each thread owns 8 consecutive columns, so
// every row read is a run of 16-byte loads.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec8;

template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    u32x4 u = *reinterpret_cast<const u32x4*>(p);
    v[0] = bf16lo(u.x); v[1] = bf16hi(u.x); v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
    v[4] = bf16lo(u.z); v[5] = bf16hi(u.z); v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 u;
    u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<u32x4*>(p) = u;
  }
};

template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const T* __restrict__ O, const int32_t* __restrict__ slot_pos,
    const float* __restrict__ w, T* __restrict__ y, int64_t Tn, int64_t d, int k, int S) {
  const int64_t t = blockIdx.x;
  const int64_t Tk = Tn * k;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < d; c += kThreads * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float v[8];
    for (int j = 0; j < k; ++j) {
      const int64_t row = slot_pos[t * k + j];
      if (row < 0) continue;  // a copy whose expert id was out of range
      const float wj = w[t * k + j];
      Vec8<T>::load(O + row * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
    }
    for (int sg = 0; sg < S; ++sg) {
      Vec8<T>::load(O + (Tk + sg * Tn + t) * d + c, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] += v[q];
    }
    Vec8<T>::store(y + t * d + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(const Shape& s, const void* expert_out, const int32_t* slot_pos,
                          const float* topk_w, void* y, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  if (s.dt == MOE_DT_BF16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, dim3((unsigned)s.T), dim3(kThreads), 0, st,
                       (const bf16_t*)expert_out, slot_pos, topk_w, (bf16_t*)y, s.T, s.d,
                       (int)s.k, (int)s.S);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)s.T), dim3(kThreads), 0, st,
                       (const float*)expert_out, slot_pos, topk_w, (float*)y, s.T, s.d,
                       (int)s.k, (int)s.S);
  return hipGetLastError();
}

}  // namespace moe
