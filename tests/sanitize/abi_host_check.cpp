// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU: every entry point is called
// with rejected arguments (no HIP call may happen) and with accepted ones,
// for which the kernel launchers below are stand-ins that record the call
// and touch no memory.  Exit status 0 when every returned status is the
// expected one; the sanitizers abort on any memory or UB error.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "moe_common.h"

namespace moe {
static int g_launches = 0;
hipError_t launch_route(const Shape&, const void*, const void*, const float*, int32_t*, float*,
                        float*, hipStream_t, void*, size_t) { ++g_launches; return hipSuccess; }
size_t route_workspace_bytes(const Shape& s) { return s.T > 64 ? 4096 : 0; }
hipError_t launch_permute(const Shape&, const int32_t*, int64_t, int32_t*, int32_t*, int32_t*,
                          int32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gate_up(const Shape&, const void*, const int32_t*, const int32_t*,
                          const void*, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_down(const Shape&, const void*, const int32_t*, const void*, void*,
                       hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_combine(const Shape&, const void*, const int32_t*, const float*, void*,
                          hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gate_up_from_ids(const Shape&, const void*, const int32_t*, const void*,
                                   void*, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  ++g_launches; return hipSuccess;
}
hipError_t launch_stream_mx(bool, const Shape&, const void*, const int32_t*, const int32_t*,
                            const uint8_t*, const uint8_t*, void*, int64_t, int64_t,
                            hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gate_up_mx_from_ids(const Shape&, const void*, const int32_t*, const uint8_t*,
                                      const uint8_t*, void*, int32_t*, int32_t*, int32_t*,
                                      int32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_balance(const Shape&, const float*, double*, double*, double*, hipStream_t) {
  ++g_launches; return hipSuccess;
}
hipError_t launch_backward(const Shape&, const void*, const void*, const void*, const void*,
                           const void*, const int32_t*, const float*, const int32_t*,
                           const int32_t*, const int32_t*, const void*, const void*, float*,
                           float*, float*, float*, float*, float*, void*, hipStream_t) {
  ++g_launches; return hipSuccess;
}
}  // namespace moe

static int g_fail = 0;
#define EXPECT(call, want)                                                            \
  do {                                                                                \
    const int got_ = (call);                                                          \
    if (got_ != (want)) {                                                             \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, \
                   got_, (int)(want));                                                \
      ++g_fail;                                                                       \
    }                                                                                 \
  } while (0)

static moe_shape shp(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k, int64_t S, int dt) {
  moe_shape s;
  s.T = T; s.d = d; s.f = f; s.E = E; s.k = k; s.n_shared = S; s.dt = dt;
  return s;
}

int main() {
  // stand-in device pointers: never dereferenced on the host
  void* p = (void*)(uintptr_t)0x10000;
  void* odd = (void*)(uintptr_t)0x10002;
  const float* fb = (const float*)p;
  const moe_shape good = shp(16, 64, 96, 8, 2, 1, MOE_DT_BF16);
  const moe_shape bad[] = {
      shp(-1, 64, 96, 8, 2, 0, 1), shp(16, 0, 96, 8, 2, 0, 1), shp(16, 12, 96, 8, 2, 0, 1),
      shp(16, 64, 20, 8, 2, 0, 1), shp(16, 64, 96, 0, 1, 0, 1), shp(16, 64, 96, 8, 0, 0, 1),
      shp(16, 64, 96, 8, 9, 0, 1), shp(16, 64, 96, 8, 2, -1, 1), shp(16, 64, 96, 8, 2, 0, 7)};
  for (const moe_shape& b : bad) {
    EXPECT(moe_route(&b, p, p, nullptr, (int32_t*)p, (float*)p, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT((int)moe_workspace_size(&b), 0);
    EXPECT(moe_layer_forward(&b, p, p, nullptr, p, p, p, p, 1u << 30, nullptr),
           MOE_ERR_INVALID_ARG);
  }
  // size limits: no overflow in any size computation
  const moe_shape huge[] = {shp(16, 1 << 30, 1 << 30, 1000, 2, 24, 1),
                            shp((int64_t)1 << 40, 64, 64, 8, 2, 0, 1),
                            shp(16, (int64_t)1 << 31, 64, 8, 2, 0, 1),
                            shp(16, 64, 96, 1024, 2, 1, 1)};
  for (const moe_shape& h : huge) {
    EXPECT(moe_route(&h, p, p, nullptr, (int32_t*)p, (float*)p, nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT((int)moe_backward_workspace_size(&h), 0);
  }
  // accepted arguments: the stand-in launchers run, nothing is dereferenced
  const size_t ws = moe_workspace_size(&good);
  size_t off[MOE_WS_COUNT];
  EXPECT(moe_workspace_offsets(&good, off), MOE_OK);
  EXPECT(moe_workspace_offsets(&good, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route(&good, p, p, fb, (int32_t*)p, (float*)p, nullptr), MOE_OK);
  EXPECT(moe_route(&good, odd, p, fb, (int32_t*)p, (float*)p, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_permute(&good, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p, (int32_t*)p,
                     nullptr), MOE_OK);
  EXPECT(moe_permute_capacity(&good, (int32_t*)p, 3, (int32_t*)p, (int32_t*)p, (int32_t*)p,
                              (int32_t*)p, nullptr), MOE_OK);
  EXPECT(moe_permute_capacity(&good, (int32_t*)p, -2, (int32_t*)p, (int32_t*)p, (int32_t*)p,
                              (int32_t*)p, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_grouped_gemm(&good, p, (int32_t*)p, (int32_t*)p, p, p, p, p, nullptr), MOE_OK);
  EXPECT(moe_combine(&good, p, (int32_t*)p, fb, p, nullptr), MOE_OK);
  EXPECT(moe_layer_forward(&good, p, p, fb, p, p, p, p, ws, nullptr), MOE_OK);
  EXPECT(moe_layer_forward(&good, p, p, fb, p, p, p, p, ws - 1, nullptr), MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward_capacity(&good, p, p, fb, p, p, 0, p, p, ws, nullptr), MOE_OK);
  const size_t bws = moe_route_balance_workspace_size(&good);
  EXPECT(moe_route_balance(&good, p, p, fb, (int32_t*)p, (float*)p, (double*)p, (double*)p, p,
                           bws, nullptr), MOE_OK);
  EXPECT(moe_route_balance(&good, p, p, fb, (int32_t*)p, (float*)p, nullptr, (double*)p, p, bws,
                           nullptr), MOE_ERR_INVALID_ARG);
  const moe_shape mx = shp(16, 64, 96, 8, 2, 1, MOE_DT_BF16);
  EXPECT(moe_layer_forward_mxfp4(&mx, p, p, fb, (uint8_t*)p, (uint8_t*)p, (uint8_t*)p,
                                 (uint8_t*)p, p, p, ws, nullptr), MOE_OK);
  const moe_shape mx_bad = shp(16, 48, 96, 8, 2, 1, MOE_DT_BF16);
  EXPECT(moe_grouped_gemm_gate_up_mxfp4(&mx_bad, p, (int32_t*)p, (int32_t*)p, (uint8_t*)p,
                                        (uint8_t*)p, p, nullptr), MOE_ERR_UNSUPPORTED);
  const size_t bw = moe_backward_workspace_size(&good);
  EXPECT(moe_layer_backward(&good, p, p, p, p, p, p, ws, (float*)p, (float*)p, (float*)p,
                            (float*)p, (float*)p, nullptr, p, bw, nullptr), MOE_OK);
  EXPECT(moe_layer_backward(&good, p, p, p, p, p, p, ws, (float*)p, (float*)p, (float*)p,
                            (float*)p, (float*)p, nullptr, p, bw - 1, nullptr), MOE_ERR_WORKSPACE);
  // no-allocation entry: oversize shapes are rejected before any HIP call
  const moe_shape big = shp(4096, 2048, 768, 128, 8, 0, MOE_DT_BF16);
  EXPECT(moe_layer_forward_static(&big, p, p, fb, p, p, p, nullptr), MOE_ERR_WORKSPACE);
  // capacity helper at its edges
  EXPECT((int)moe_expert_capacity(4096, 8, 128, 1.25), 320);
  EXPECT((int)moe_expert_capacity(1, 1, 1, std::nan("")), -1);
  EXPECT((int)moe_expert_capacity(1, 1, 1, std::numeric_limits<double>::infinity()), -1);
  EXPECT((int)moe_expert_capacity(std::numeric_limits<int64_t>::max(), 64, 1, 1e9), -1);
  for (int st = -1; st < 6; ++st)
    if (!moe_status_string(st) || !std::strlen(moe_status_string(st))) ++g_fail;
  if (moe::g_launches == 0) ++g_fail;
  std::printf("%s: %d launches recorded, %d failures\n", g_fail ? "FAIL" : "ok", moe::g_launches,
              g_fail);
  return g_fail ? 1 : 0;
}
