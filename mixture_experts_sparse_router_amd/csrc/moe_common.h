// moe_common.h -- internal helpers shared by the HIP sources of libmoe.
// (Not part of the public ABI; the public header is include/moe.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ------------------------------------------------------------------ types

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern in memory

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Low / high bfloat16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero_unless(bool ok, u32x4 v) {
  return u32x4{ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u};
}

// D = A * B + C on a 16x16x32 bf16 tile (fp32 accumulate).  Lane l supplies
// A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16]; it receives
// D[4*(l/16) + q][l%16] in element q.
__device__ __forceinline__ f32x4 mfma16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ------------------------------------------------ global -> LDS copies
// Buffer resource word 3 for raw (untyped, stride 0) buffers on gfx9-family
// parts: 32-bit data format; the range check is then "offset >= num_records".
constexpr int kRsrcWord3 = 0x00020000;
// A byte offset that fails the range check of every resource used here
// (each spans at most 2^31 bytes; see the launcher).
constexpr uint32_t kOOB = 0x80000000u;

// Global -> LDS copy of 16 bytes per lane: lane l of the wave writes
// lds + 16*l with bytes [voff, voff+16) of the resource (zeros if out of
// range).  The LDS address goes through an integer that alias analysis
// cannot follow, so the compiler does not try to match copies in flight to
// the LDS reads that follow (it would wait for all of them); the ring's
// readers are ordered after the copies they need by the explicit vmcnt wait
// and barrier of every K tile.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform
  asm("" : "+s"(lds));                        // opaque; emits no instruction
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)(uintptr_t)lds, 16, (int)voff, 0, 0, 0);
}

// D = A * B + C on a 32x32x16 bf16 tile (fp32 accumulate).
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// silu(z) * u in fp32.  silu(z) = z / (1 + e^-z).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// --------------------------------------------------------- token of a row
// Row r of the permuted buffers belongs to token sorted_slot[r] / k for the
// routed rows r < T*k, and to token (r - T*k) % T for the shared rows.  Every
// quantity is below 2^31 (R < 2^31), so the divisions are 32-bit.
__device__ __forceinline__ int64_t token_of(int64_t r, int32_t slot, int64_t Tk, int64_t k,
                                            int64_t T) {
  return r < Tk ? (int64_t)((uint32_t)slot / (uint32_t)k)
                : (int64_t)((uint32_t)(r - Tk) % (uint32_t)T);
}
__device__ __forceinline__ int64_t row_token(int64_t r, const int32_t* sorted_slot,
                                             int64_t Tk, int64_t k, int64_t T) {
  return token_of(r, r < Tk ? sorted_slot[r] : 0, Tk, k, T);
}

// ----------------------------------------------------------- host helpers

struct Shape {
  int64_t T, d, f, E, k, S;
  int dt;
  int64_t Tk() const { return T * k; }
  int64_t R() const { return T * k + S * T; }
  int64_t G() const { return E + S; }  // expert groups
};

inline Shape to_shape(const moe_shape* s) {
  return Shape{s->T, s->d, s->f, s->E, s->k, s->n_shared, (int)s->dt};
}

// Launchers (return hipSuccess or the launch error).  Argument checking is
// done by the ABI layer before any of these is called.
// logits_out: NULL, or [T, E] fp32 that receives the logits (bias included).
// scratch: NULL, or device memory (256-byte aligned) that the router may use
// for partial sums until it returns to the stream (large bf16 batches).
hipError_t launch_route(const Shape& s, const void* x, const void* W_router,
                        const float* bias, int32_t* topk_idx, float* topk_w,
                        float* logits_out, hipStream_t st, void* scratch = nullptr,
                        size_t scratch_bytes = 0);
// Scratch bytes with which launch_route takes its fastest path for this
// shape (0: it needs none).
size_t route_workspace_bytes(const Shape& s);
// capacity < 0: none.
hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int64_t capacity,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                          int32_t* slot_pos, hipStream_t st);
// MXFP4 expert weights (Wq packed FP4, Ws E8M0 scales), T <= 64, bf16
// activations; gated selects the gate_up form.  K % 32 == 0.
hipError_t launch_stream_mx(bool gated, const Shape& s, const void* A,
                            const int32_t* sorted_slot, const int32_t* offsets,
                            const uint8_t* Wq, const uint8_t* Ws, void* out, int64_t K,
                            int64_t N, hipStream_t st);
// Decode-sized batches (T <= 64): the MXFP4 gate_up with the group rows found
// from the expert ids, writing the permutation on the way.
hipError_t launch_gate_up_mx_from_ids(const Shape& s, const void* x, const int32_t* topk_idx,
                                      const uint8_t* Wq, const uint8_t* Ws, void* act,
                                      int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                                      int32_t* slot_pos, hipStream_t st);
// Backward pass (bf16): workspace layout and the launch sequence; the
// forward's routing, permutation, act and expert_out are inputs.
// Workspace (bytes, 256-aligned pieces): dO [R, d] bf16, H [R, 2f] fp32,
// dA [R, f] fp32, dH [R, 2f] bf16, dXp [R, d] fp32, dl [T, k] fp32, router
// partials [kRouterChunks, E, d] + [kRouterChunks, E] fp32.
constexpr int kRouterChunks = 32;
inline size_t bwd_layout(const Shape& s, size_t* off) {
  const size_t R = (size_t)s.R(), d = (size_t)s.d, f = (size_t)s.f;
  const size_t sizes[7] = {R * d * 2,  R * 2 * f * 4, R * f * 4, R * 2 * f * 2,
                           R * d * 4,  (size_t)s.Tk() * 4,
                           (size_t)kRouterChunks * (size_t)s.E * (d + 1) * 4};
  size_t at = 0;
  for (int i = 0; i < 7; ++i) {
    off[i] = at;
    at += (sizes[i] + 255) & ~(size_t)255;
  }
  return at;
}
hipError_t launch_backward(const Shape& s, const void* x, const void* W_router,
                           const void* W_gate_up, const void* W_down, const void* dy,
                           const int32_t* topk_idx, const float* topk_w,
                           const int32_t* offsets, const int32_t* sorted_slot,
                           const int32_t* slot_pos, const void* act, const void* expert_out,
                           float* dx, float* dWr, float* db, float* dWgu, float* dWd, float* dw,
                           void* workspace, hipStream_t st);
// Router load statistics from the logits: importance[E] (mean softmax
// probability) and the balance loss; partial holds balance_partials(T) * E
// doubles (one row per workgroup of kBalTokens tokens).
constexpr int kBalTokens = 16;
inline int64_t balance_partials(int64_t T) { return (T + kBalTokens - 1) / kBalTokens; }
hipError_t launch_balance(const Shape& s, const float* logits, double* partial,
                          double* importance, double* loss, hipStream_t st);
hipError_t launch_gate_up(const Shape& s, const void* x, const int32_t* sorted_slot,
                          const int32_t* offsets, const void* W_gate_up, void* act,
                          hipStream_t st);
// bf16: the gate_up GEMM's pre-activation values, H [R, 2f] fp32 (gate in
// columns < f, up in f + c), for the backward pass.
hipError_t launch_gate_up_preact(const Shape& s, const void* x, const int32_t* sorted_slot,
                                 const int32_t* offsets, const void* W_gate_up, float* H,
                                 hipStream_t st);
// Decode-sized groups (T <= 64), bf16 only; gated selects the gate_up form.
hipError_t launch_stream_gemm(bool gated, const Shape& s, const void* A,
                              const int32_t* sorted_slot, const int32_t* offsets, const void* W,
                              void* out, int64_t K, int64_t N, hipStream_t st);
// Decode-sized batches (T <= 64, bf16): the gate_up GEMM's pre-activation
// values H [R, 2f] fp32 (as launch_gate_up_preact), streaming kernel.
hipError_t launch_stream_gate_up_preact(const Shape& s, const void* x, const int32_t* sorted_slot,
                                        const int32_t* offsets, const void* W_gate_up, float* H,
                                        hipStream_t st);
// Decode-sized batches (T <= 64, bf16): gate_up with the group rows found
// from the expert ids, writing the permutation on the way.
hipError_t launch_gate_up_from_ids(const Shape& s, const void* x, const int32_t* topk_idx,
                                   const void* W_gate_up, void* act, int32_t* counts,
                                   int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                                   hipStream_t st);
hipError_t launch_down(const Shape& s, const void* act, const int32_t* offsets,
                       const void* W_down, void* expert_out, hipStream_t st);
hipError_t launch_combine(const Shape& s, const void* expert_out,
                          const int32_t* slot_pos, const float* topk_w, void* y,
                          hipStream_t st);

}  // namespace moe
