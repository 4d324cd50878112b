// abi.hip -- the C entry points of libmoe: argument checks, workspace layout
// and the stream-ordered launch sequence of the layer.  The steps and where
// the pages define them are documented in include/moe.h.
#include <math.h>
#include <string.h>

#include <atomic>

#include "moe_common.h"

using namespace moe;

// Intermediates of moe_layer_forward_static: one array per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
// device address of `scratch` on each device, looked up on first use there
std::atomic<void*> g_scratch_ptr[kMaxDevices];

constexpr int64_t kMaxGroups = 1024;
constexpr int64_t kMaxK = 64;
constexpr int64_t kMaxRows = (int64_t)1 << 31;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Non-null and 16-byte aligned, unless the tensor is empty.
inline bool ok_ptr(const void* p, int64_t elems) {
  if (elems == 0) return true;
  return p != nullptr && aligned16(p);
}

inline int64_t esize(const Shape& s) { return s.dt == MOE_DT_BF16 ? 2 : 4; }

int check_shape(const moe_shape* m) {
  if (!m) return MOE_ERR_INVALID_ARG;
  if (m->T < 0 || m->d < 1 || m->f < 1 || m->E < 1 || m->k < 1 || m->k > m->E ||
      m->n_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (m->dt != MOE_DT_F32 && m->dt != MOE_DT_BF16) return MOE_ERR_INVALID_ARG;
  if (m->d % 8 != 0 || m->f % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (m->E + m->n_shared > kMaxGroups) return MOE_ERR_UNSUPPORTED;
  if (m->k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (m->d > ((int64_t)1 << 30) || m->f > ((int64_t)1 << 30)) return MOE_ERR_UNSUPPORTED;
  // element counts of the weight tensors, (E+S) * 2f * d, stay below 2^62
  if (m->d * m->f > ((int64_t)1 << 60) / (m->E + m->n_shared)) return MOE_ERR_UNSUPPORTED;
  if (m->T >= kMaxRows / (m->k + m->n_shared)) return MOE_ERR_UNSUPPORTED;  // R < 2^31
  // bf16 batches past decode size: the tiled GEMM addresses x and one
  // expert's weights with 32-bit byte offsets below 2^31
  if (m->dt == MOE_DT_BF16 && m->T > 64 &&
      (m->T * m->d >= ((int64_t)1 << 30) || m->f * m->d >= ((int64_t)1 << 29)))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Shapes of the MXFP4 entry points: bf16 activations, decode-sized batches,
// d and f multiples of the 32-element scale block.
int check_mxfp4_shape(const moe_shape* m) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  if (m->dt != MOE_DT_BF16 || m->T > 64 || m->d % 32 != 0 || m->f % 32 != 0)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Tensors of the whole-layer entry points.
int check_layer_ptrs(const Shape& s, const void* x, const void* W_router, const float* bias,
                     const void* W_gate_up, const void* W_down, const void* y) {
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) ||
      !ok_ptr(W_gate_up, s.G() * 2 * s.f * s.d) || !ok_ptr(W_down, s.G() * s.d * s.f) ||
      !ok_ptr(y, s.T * s.d))
    return MOE_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

thread_local hipError_t g_last_hip_error = hipSuccess;

inline int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = e;
  return MOE_ERR_HIP;
}

inline size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace of moe_route_balance: logits [T, E] fp32, then the per-block
// partial importances [balance_partials(T), E] fp64.
size_t balance_layout(const Shape& s, size_t* logits_off, size_t* partial_off) {
  *logits_off = 0;
  *partial_off = round_up((size_t)s.T * (size_t)s.E * 4);
  return *partial_off + round_up((size_t)balance_partials(s.T) * (size_t)s.E * 8);
}

void layout(const Shape& s, size_t* off, size_t* total) {
  const size_t Tk = (size_t)s.Tk();
  const size_t R = (size_t)s.R();
  const size_t G = (size_t)s.G();
  const size_t sizes[MOE_WS_COUNT] = {
      Tk * 4, Tk * 4, G * 4, (G + 1) * 4, Tk * 4, Tk * 4,
      R * (size_t)s.f * (size_t)esize(s), R * (size_t)s.d * (size_t)esize(s)};
  size_t at = 0;
  for (int i = 0; i < MOE_WS_COUNT; ++i) {
    off[i] = at;
    at += round_up(sizes[i]);
  }
  *total = at;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_version(void) { return "moe-gfx950 1.0"; }

const char* moe_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

size_t moe_workspace_size(const moe_shape* m) {
  if (check_shape(m) != MOE_OK) return 0;
  size_t off[MOE_WS_COUNT], total;
  layout(to_shape(m), off, &total);
  return total;
}

int moe_workspace_offsets(const moe_shape* m, size_t* out) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  if (!out) return MOE_ERR_INVALID_ARG;
  size_t total;
  layout(to_shape(m), out, &total);
  return MOE_OK;
}

int moe_route(const moe_shape* m, const void* x, const void* W_router, const float* bias,
              int32_t* topk_idx, float* topk_w, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) ||
      !ok_ptr(topk_idx, s.Tk()) || !ok_ptr(topk_w, s.Tk()))
    return MOE_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_route(s, x, W_router, bias, topk_idx, topk_w, nullptr, (hipStream_t)stream));
}

size_t moe_route_workspace_size(const moe_shape* m) {
  if (check_shape(m) != MOE_OK) return 0;
  return route_workspace_bytes(to_shape(m));
}

int moe_route_ws(const moe_shape* m, const void* x, const void* W_router, const float* bias,
                 int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) ||
      !ok_ptr(topk_idx, s.Tk()) || !ok_ptr(topk_w, s.Tk()))
    return MOE_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return MOE_ERR_INVALID_ARG;
  const size_t need = route_workspace_bytes(s);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE;
  if (need > 0 && (!workspace || ((uintptr_t)workspace & 255u))) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(s, x, W_router, bias, topk_idx, topk_w, nullptr,
                                 (hipStream_t)stream, need > 0 ? workspace : nullptr,
                                 workspace_bytes));
}

size_t moe_route_balance_workspace_size(const moe_shape* m) {
  if (check_shape(m) != MOE_OK) return 0;
  size_t lo, part;
  return balance_layout(to_shape(m), &lo, &part);
}

int moe_route_balance(const moe_shape* m, const void* x, const void* W_router,
                      const float* bias, int32_t* topk_idx, float* topk_w, double* importance,
                      double* loss, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) ||
      !ok_ptr(topk_idx, s.Tk()) || !ok_ptr(topk_w, s.Tk()) || !ok_ptr(importance, s.E) ||
      !ok_ptr(loss, 1))
    return MOE_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return MOE_ERR_INVALID_ARG;
  size_t lo_off, part_off;
  const size_t total = balance_layout(s, &lo_off, &part_off);
  if (workspace_bytes < total) return MOE_ERR_WORKSPACE;
  if (total > 0 && (!workspace || ((uintptr_t)workspace & 255u))) return MOE_ERR_INVALID_ARG;
  char* ws = (char*)workspace;
  float* lg = total ? (float*)(ws + lo_off) : nullptr;
  double* part = total ? (double*)(ws + part_off) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_route(s, x, W_router, bias, topk_idx, topk_w, lg, st);
  if (e == hipSuccess) e = launch_balance(s, lg, part, importance, loss, st);
  return hip_status(e);
}

int moe_permute_capacity(const moe_shape* m, const int32_t* topk_idx, int64_t capacity,
                         int32_t* counts, int32_t* offsets, int32_t* sorted_slot,
                         int32_t* slot_pos, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(topk_idx, s.Tk()) || !ok_ptr(counts, s.G()) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(sorted_slot, s.Tk()) || !ok_ptr(slot_pos, s.Tk()))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_permute(s, topk_idx, capacity, counts, offsets, sorted_slot,
                                   slot_pos, (hipStream_t)stream));
}

int moe_permute(const moe_shape* m, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(topk_idx, s.Tk()) || !ok_ptr(counts, s.G()) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(sorted_slot, s.Tk()) || !ok_ptr(slot_pos, s.Tk()))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_permute(s, topk_idx, -1, counts, offsets, sorted_slot, slot_pos,
                                   (hipStream_t)stream));
}

int64_t moe_expert_capacity(int64_t T, int64_t k, int64_t E, double capacity_factor) {
  if (T < 0 || k < 1 || E < 1 || !(capacity_factor >= 0.0) || capacity_factor > 1e9)
    return -1;
  // T * k in double: exact below 2^53 copies, and no integer overflow above
  const double c = ceil(capacity_factor * ((double)T * (double)k) / (double)E);
  return c < 4.0e18 ? (int64_t)c : -1;
}

int moe_grouped_gemm_gate_up(const moe_shape* m, const void* x, const int32_t* sorted_slot,
                             const int32_t* offsets, const void* W_gate_up, void* act,
                             void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(sorted_slot, s.Tk()) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(W_gate_up, s.G() * 2 * s.f * s.d) || !ok_ptr(act, s.R() * s.f))
    return MOE_ERR_INVALID_ARG;
  return hip_status(
      launch_gate_up(s, x, sorted_slot, offsets, W_gate_up, act, (hipStream_t)stream));
}

int moe_grouped_gemm_down(const moe_shape* m, const void* act, const int32_t* offsets,
                          const void* W_down, void* expert_out, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(act, s.R() * s.f) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(W_down, s.G() * s.d * s.f) || !ok_ptr(expert_out, s.R() * s.d))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_down(s, act, offsets, W_down, expert_out, (hipStream_t)stream));
}

int moe_grouped_gemm(const moe_shape* m, const void* x, const int32_t* sorted_slot,
                     const int32_t* offsets, const void* W_gate_up, const void* W_down,
                     void* act, void* expert_out, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(sorted_slot, s.Tk()) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(W_gate_up, s.G() * 2 * s.f * s.d) || !ok_ptr(W_down, s.G() * s.d * s.f) ||
      !ok_ptr(act, s.R() * s.f) || !ok_ptr(expert_out, s.R() * s.d))
    return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_gate_up(s, x, sorted_slot, offsets, W_gate_up, act, st);
  if (e == hipSuccess) e = launch_down(s, act, offsets, W_down, expert_out, st);
  return hip_status(e);
}

int moe_combine(const moe_shape* m, const void* expert_out, const int32_t* slot_pos,
                const float* topk_w, void* y, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(expert_out, s.R() * s.d) || !ok_ptr(slot_pos, s.Tk()) ||
      !ok_ptr(topk_w, s.Tk()) || !ok_ptr(y, s.T * s.d))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(s, expert_out, slot_pos, topk_w, y, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The layer, with an expert capacity (capacity < 0: none).
int layer_forward(const moe_shape* m, const void* x, const void* W_router, const float* bias,
                  const void* W_gate_up, const void* W_down, int64_t capacity, void* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  rc = check_layer_ptrs(s, x, W_router, bias, W_gate_up, W_down, y);
  if (rc != MOE_OK) return rc;
  size_t off[MOE_WS_COUNT], total;
  layout(s, off, &total);
  if (workspace_bytes < total) return MOE_ERR_WORKSPACE;
  if (total > 0 && (!workspace || ((uintptr_t)workspace & 255u))) return MOE_ERR_INVALID_ARG;
  if (s.T == 0) return MOE_OK;

  char* ws = (char*)workspace;
  int32_t* idx = (int32_t*)(ws + off[MOE_WS_TOPK_IDX]);
  float* w = (float*)(ws + off[MOE_WS_TOPK_W]);
  int32_t* counts = (int32_t*)(ws + off[MOE_WS_COUNTS]);
  int32_t* offsets = (int32_t*)(ws + off[MOE_WS_OFFSETS]);
  int32_t* sorted_slot = (int32_t*)(ws + off[MOE_WS_SORTED_SLOT]);
  int32_t* slot_pos = (int32_t*)(ws + off[MOE_WS_SLOT_POS]);
  void* act = ws + off[MOE_WS_ACT];
  void* out = ws + off[MOE_WS_EXPERT_OUT];

  hipStream_t st = (hipStream_t)stream;
  // act and expert_out (the workspace's last two regions) are written only
  // after the router: it may keep partial sums there
  hipError_t e = launch_route(s, x, W_router, bias, idx, w, nullptr, st, act,
                              total - off[MOE_WS_ACT]);
  if (s.dt == MOE_DT_BF16 && s.T <= 64 && capacity < 0) {
    // decode batches: the gate_up kernel finds its rows from the ids and
    // writes the permutation itself (one launch fewer)
    if (e == hipSuccess)
      e = launch_gate_up_from_ids(s, x, idx, W_gate_up, act, counts, offsets, sorted_slot,
                                  slot_pos, st);
  } else {
    if (e == hipSuccess)
      e = launch_permute(s, idx, capacity, counts, offsets, sorted_slot, slot_pos, st);
    if (e == hipSuccess) e = launch_gate_up(s, x, sorted_slot, offsets, W_gate_up, act, st);
  }
  if (e == hipSuccess) e = launch_down(s, act, offsets, W_down, out, st);
  if (e == hipSuccess) e = launch_combine(s, out, slot_pos, w, y, st);
  return hip_status(e);
}

}  // namespace

extern "C" {

int moe_layer_forward(const moe_shape* m, const void* x, const void* W_router,
                      const float* bias, const void* W_gate_up, const void* W_down, void* y,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return layer_forward(m, x, W_router, bias, W_gate_up, W_down, -1, y, workspace,
                       workspace_bytes, stream);
}

int moe_layer_forward_capacity(const moe_shape* m, const void* x, const void* W_router,
                               const float* bias, const void* W_gate_up, const void* W_down,
                               int64_t capacity, void* y, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  return layer_forward(m, x, W_router, bias, W_gate_up, W_down, capacity, y, workspace,
                       workspace_bytes, stream);
}

int moe_grouped_gemm_gate_up_mxfp4(const moe_shape* m, const void* x,
                                   const int32_t* sorted_slot, const int32_t* offsets,
                                   const uint8_t* Wq_gate_up, const uint8_t* Ws_gate_up,
                                   void* act, void* stream) {
  int rc = check_mxfp4_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(sorted_slot, s.Tk()) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(Wq_gate_up, s.G() * 2 * s.f * s.d / 2) || !ok_ptr(Ws_gate_up, s.G() * 2 * s.f) ||
      !ok_ptr(act, s.R() * s.f))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_stream_mx(true, s, x, sorted_slot, offsets, Wq_gate_up, Ws_gate_up,
                                     act, s.d, s.f, (hipStream_t)stream));
}

int moe_grouped_gemm_down_mxfp4(const moe_shape* m, const void* act, const int32_t* offsets,
                                const uint8_t* Wq_down, const uint8_t* Ws_down,
                                void* expert_out, void* stream) {
  int rc = check_mxfp4_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(act, s.R() * s.f) || !ok_ptr(offsets, s.G() + 1) ||
      !ok_ptr(Wq_down, s.G() * s.d * s.f / 2) || !ok_ptr(Ws_down, s.G() * s.d) ||
      !ok_ptr(expert_out, s.R() * s.d))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_stream_mx(false, s, act, nullptr, offsets, Wq_down, Ws_down,
                                     expert_out, s.f, s.d, (hipStream_t)stream));
}

int moe_layer_forward_mxfp4(const moe_shape* m, const void* x, const void* W_router,
                            const float* bias, const uint8_t* Wq_gate_up,
                            const uint8_t* Ws_gate_up, const uint8_t* Wq_down,
                            const uint8_t* Ws_down, void* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = check_mxfp4_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) || !ok_ptr(y, s.T * s.d) ||
      !ok_ptr(Wq_gate_up, s.G() * 2 * s.f * s.d / 2) || !ok_ptr(Ws_gate_up, s.G() * 2 * s.f) ||
      !ok_ptr(Wq_down, s.G() * s.d * s.f / 2) || !ok_ptr(Ws_down, s.G() * s.d))
    return MOE_ERR_INVALID_ARG;
  if (bias && ((uintptr_t)bias & 3u)) return MOE_ERR_INVALID_ARG;
  size_t off[MOE_WS_COUNT], total;
  layout(s, off, &total);
  if (workspace_bytes < total) return MOE_ERR_WORKSPACE;
  if (total > 0 && (!workspace || ((uintptr_t)workspace & 255u))) return MOE_ERR_INVALID_ARG;
  if (s.T == 0) return MOE_OK;
  char* ws = (char*)workspace;
  int32_t* idx = (int32_t*)(ws + off[MOE_WS_TOPK_IDX]);
  float* w = (float*)(ws + off[MOE_WS_TOPK_W]);
  int32_t* counts = (int32_t*)(ws + off[MOE_WS_COUNTS]);
  int32_t* offsets = (int32_t*)(ws + off[MOE_WS_OFFSETS]);
  int32_t* sorted_slot = (int32_t*)(ws + off[MOE_WS_SORTED_SLOT]);
  int32_t* slot_pos = (int32_t*)(ws + off[MOE_WS_SLOT_POS]);
  void* act = ws + off[MOE_WS_ACT];
  void* out = ws + off[MOE_WS_EXPERT_OUT];
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_route(s, x, W_router, bias, idx, w, nullptr, st);
  // the gate_up kernel finds its rows from the ids and writes the
  // permutation (one launch fewer, as in the bf16 decode layer)
  if (e == hipSuccess)
    e = launch_gate_up_mx_from_ids(s, x, idx, Wq_gate_up, Ws_gate_up, act, counts, offsets,
                                   sorted_slot, slot_pos, st);
  if (e == hipSuccess)
    e = launch_stream_mx(false, s, act, nullptr, offsets, Wq_down, Ws_down, out, s.f, s.d, st);
  if (e == hipSuccess) e = launch_combine(s, out, slot_pos, w, y, st);
  return hip_status(e);
}

size_t moe_backward_workspace_size(const moe_shape* m) {
  if (check_shape(m) != MOE_OK || m->dt != MOE_DT_BF16) return 0;
  size_t off[7];
  return bwd_layout(to_shape(m), off);
}

int moe_layer_backward(const moe_shape* m, const void* x, const void* W_router,
                       const void* W_gate_up, const void* W_down, const void* dy,
                       const void* fwd_workspace, size_t fwd_workspace_bytes, float* dx,
                       float* dW_router, float* db, float* dW_gate_up, float* dW_down,
                       float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  if (m->dt != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  const Shape s = to_shape(m);
  if (!ok_ptr(x, s.T * s.d) || !ok_ptr(W_router, s.E * s.d) ||
      !ok_ptr(W_gate_up, s.G() * 2 * s.f * s.d) || !ok_ptr(W_down, s.G() * s.d * s.f) ||
      !ok_ptr(dy, s.T * s.d) || !ok_ptr(dx, s.T * s.d) || !ok_ptr(dW_router, s.E * s.d) ||
      !ok_ptr(db, s.E) || !ok_ptr(dW_gate_up, s.G() * 2 * s.f * s.d) ||
      !ok_ptr(dW_down, s.G() * s.d * s.f) || (dw && !aligned16(dw)))
    return MOE_ERR_INVALID_ARG;
  size_t foff[MOE_WS_COUNT], ftotal;
  layout(s, foff, &ftotal);
  if (fwd_workspace_bytes < ftotal) return MOE_ERR_WORKSPACE;
  if (ftotal > 0 && (!fwd_workspace || ((uintptr_t)fwd_workspace & 255u)))
    return MOE_ERR_INVALID_ARG;
  size_t boff[7];
  const size_t btotal = bwd_layout(s, boff);
  if (workspace_bytes < btotal) return MOE_ERR_WORKSPACE;
  if (btotal > 0 && (!workspace || ((uintptr_t)workspace & 255u))) return MOE_ERR_INVALID_ARG;
  const char* fw = (const char*)fwd_workspace;
  return hip_status(launch_backward(
      s, x, W_router, W_gate_up, W_down, dy, (const int32_t*)(fw + foff[MOE_WS_TOPK_IDX]),
      (const float*)(fw + foff[MOE_WS_TOPK_W]), (const int32_t*)(fw + foff[MOE_WS_OFFSETS]),
      (const int32_t*)(fw + foff[MOE_WS_SORTED_SLOT]),
      (const int32_t*)(fw + foff[MOE_WS_SLOT_POS]), fw + foff[MOE_WS_ACT],
      fw + foff[MOE_WS_EXPERT_OUT], dx, dW_router, db, dW_gate_up, dW_down, dw, workspace,
      (hipStream_t)stream));
}

int moe_layer_forward_static(const moe_shape* m, const void* x, const void* W_router,
                             const float* bias, const void* W_gate_up, const void* W_down,
                             void* y, void* stream) {
  int rc = check_shape(m);
  if (rc != MOE_OK) return rc;
  const Shape s = to_shape(m);
  rc = check_layer_ptrs(s, x, W_router, bias, W_gate_up, W_down, y);
  if (rc != MOE_OK) return rc;
  size_t off[MOE_WS_COUNT], total;
  layout(s, off, &total);
  if (total > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  if (s.T == 0) return MOE_OK;
  // the calling thread's current device: look up (once) where its copy of
  // the array lives
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* ws = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ws) {
    e = hipGetSymbolAddress(&ws, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!ws) return MOE_ERR_HIP;
    g_scratch_ptr[dev].store(ws, std::memory_order_release);
  }
  return moe_layer_forward(m, x, W_router, bias, W_gate_up, W_down, y, ws,
                           (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}

}  // extern "C"
