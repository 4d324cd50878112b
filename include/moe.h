/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE feed-forward layer library.
 *
 * One sparse-routed Mixture-of-Experts FFN layer, forward pass, in five steps:
 *
 *   1. router logits      L[t,e] = sum_i x[t,i] W_router[e,i] (+ bias[e])
 *   2. routing            softmax over the E experts, the k largest taken
 *                         (ties to the lower expert index), their
 *                         probabilities renormalised to sum to one
 *   3. permutation        token copies grouped by expert: per-expert
 *                         histogram, exclusive prefix sum, stable scatter
 *   4. expert FFN         grouped GEMMs over the variable-size groups:
 *                         act = silu(x W_gate^T) * (x W_up^T), out = act W_down^T
 *   5. combine            y[t] = sum_j w[t,j] out[copy (t,j)] (+ shared experts)
 *
 * Where the pages define each step:
 *   - router = small linear layer scoring every expert, then softmax and
 *     top-k: Baidu "MoE稀疏架构是什么" page, section 三.1 and the section 四
 *     pseudocode; qqiyuan 2026 MoE guide, MoELayer pseudocode; yunthe
 *     "分工的艺术" page, section 1.1;
 *   - renormalised top-k weights and the weighted sum over the selected
 *     experts only: Baidu page, section 四;
 *   - sort tokens by expert id, group them, one grouped GEMM, then apply the
 *     routing weights and gather/reorder back: aitoday "MoEs in
 *     Transformers" page, section "Expert Backend" (grouped_mm);
 *   - packed expert weights, gate_up_proj [E, 2f, d] (w1 rows then w3 rows)
 *     and down_proj [E, d, f]: aitoday page, section "Dynamic Weight Loading
 *     with WeightConverter".
 * The expert function (SwiGLU), the tie rule, shared experts and the router
 * bias are readings where the pages are silent; they are stated at each call.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library allocates and frees nothing and carries no data between calls
 *     (it only caches per-device configuration: the CU count and one kernel
 *     attribute, set on first use).
 *   - Tensors are dense row-major, last dimension contiguous, 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls only enqueue work; results are valid once the stream is
 *     synchronised.  No call synchronises the host.
 *   - Arguments are checked on the host before any HIP call; a rejected call
 *     enqueues nothing.  Launch failures are reported as MOE_ERR_HIP.
 *   - Element type: dt = MOE_DT_BF16 (bfloat16) or MOE_DT_F32 (binary32) for
 *     x, W_router, W_gate_up, W_down, act, expert_out and y alike.  Routing
 *     weights are always float32, indices int32.
 *   - Numerics: router logits are accumulated in fp64 (for bf16 batches of
 *     more than 64 tokens, only for the experts that a bf16 screen with a
 *     proven error bound cannot rule out; selection and weights are the
 *     same as with fp64 everywhere); GEMMs multiply in dt
 *     and accumulate in fp32; act and expert_out are rounded to dt (round to
 *     nearest even); the combine accumulates in fp32 in a fixed order, so
 *     repeated calls are bitwise identical.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad size, null or misaligned pointer       */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the library handles */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_size  */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed         */
} moe_status;

typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 } moe_dtype;

/* Layer shape.
 *   T        tokens (rows of x), T >= 0
 *   d        model dimension, multiple of 8
 *   f        expert FFN dimension, multiple of 8
 *   E        routed experts, 1 <= E
 *   k        experts per token, 1 <= k <= E
 *   n_shared always-on shared experts S >= 0 with E + S <= 1024; they are
 *            stored after the routed experts in W_gate_up / W_down, get
 *            weight 1 for every token and take no part in the softmax
 *   dt       moe_dtype of the float tensors
 * Derived: R = T*k + S*T rows of the permuted buffers; R < 2^31.
 * bf16 with T > 64 also needs T*d < 2^30 and f*d < 2^29 (x and one expert's
 * gate_up weights each under 2 GiB); other shapes get MOE_ERR_UNSUPPORTED. */
typedef struct {
  int64_t T, d, f, E, k, n_shared;
  int32_t dt;
} moe_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int status);

/* Library version string, e.g. "moe-gfx950 1.0". */
const char* moe_version(void);

/* Text of the last HIP error an entry point of this library met on the
 * calling thread ("no error" if none); use it after MOE_ERR_HIP. */
const char* moe_last_hip_error(void);

/* ---------------------------------------------------------------- step 1+2
 * moe_route: router logits and top-k routing of every token.
 *   x         [T, d]  dt
 *   W_router  [E, d]  dt
 *   bias      [E] float32 added to the logits, or NULL (reading: used only
 *             to give a router prior, e.g. a Zipf-skewed load)
 *   topk_idx  [T, k]  int32 out: slot j of token t holds its rank-j expert
 *             (larger logit first; equal logits, lower index first)
 *   topk_w    [T, k]  float32 out: softmax probabilities of the selected
 *             experts renormalised over the k of them (each row sums to 1)
 * Logits are accumulated in fp64 and ranked in fp64. */
int moe_route(const moe_shape* s, const void* x, const void* W_router,
              const float* bias, int32_t* topk_idx, float* topk_w,
              void* stream);

/* moe_route_ws: moe_route with a workspace for the router's partial sums.
 * Same steps and results (selection and weights); large bf16 batches with
 * few experts or a large router matrix route faster with it: the screen runs
 * as a K-split product over tiles of 64 or 128 tokens, whose fp64 partials
 * the workspace holds, then a selection pass.  moe_layer_forward does the
 * same inside its own workspace.
 *   workspace  moe_route_workspace_size(s) bytes, 256-byte aligned (NULL
 *              when the size is 0); MOE_ERR_WORKSPACE if smaller; it holds
 *              nothing of use after the call. */
size_t moe_route_workspace_size(const moe_shape* s);

int moe_route_ws(const moe_shape* s, const void* x, const void* W_router,
                 const float* bias, int32_t* topk_idx, float* topk_w,
                 void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------- router load statistics
 * moe_route_balance: moe_route plus the router's load statistics and the
 * load-balance loss (yunthe "分工的艺术" page, section 3.1, load balance
 * loss: the gate averaged over the batch, compared with the uniform
 * distribution by KL divergence, batch-mean reduced; the gate is the
 * softmax over all experts, that page's section 1.1 gating code).
 *   topk_idx, topk_w  as moe_route (same values)
 *   importance [E] float64 out: imp_e = (1/T) sum_t softmax(L_t)_e, the
 *              softmax over all E experts of token t's logits (bias
 *              included); T = 0 gives NaN
 *   loss       [1] float64 out:
 *              (1/E) sum_e (1/E) (log(1/E) - log(imp_e + 1e-8))
 *   workspace  device memory of moe_route_balance_workspace_size(s) bytes,
 *              256-byte aligned (the logits and per-block partial sums)
 * Numerics: the logits enter the softmax rounded to fp32; every expert that
 * can be selected has its exact fp64 logit, and on the bf16 screen path
 * (more than 64 tokens) the others have the screen's estimate, within
 * 2^-14 * ||x_t|| * ||w_e|| of the exact logit.  exp in fp32, sums in fp64 in
 * a fixed order (repeated calls are bitwise identical). */
size_t moe_route_balance_workspace_size(const moe_shape* s);

int moe_route_balance(const moe_shape* s, const void* x, const void* W_router,
                      const float* bias, int32_t* topk_idx, float* topk_w,
                      double* importance, double* loss, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ step 3
 * moe_permute: group the T*k token copies by expert.
 * Copy s = t*k + j goes to expert topk_idx[s].
 *   counts      [E+S]   int32 out: copies per expert; every shared expert
 *               counts T
 *   offsets     [E+S+1] int32 out: exclusive prefix sum of counts
 *               (offsets[E] = T*k, offsets[E+S] = R)
 *   sorted_slot [T*k]   int32 out: row r < T*k of the permuted buffers holds
 *               copy sorted_slot[r]; inside one expert the copies are in
 *               ascending s (stable).  Rows T*k + sigma*T + t (shared expert
 *               sigma, token t) are implicit and not stored.
 *   slot_pos    [T*k]   int32 out: inverse map, row of copy s
 * topk_idx entries should lie in [0, E).  A copy whose id lies outside it
 * selects no expert: it is dropped.  Dropped copies take the first rows,
 * [0, D), in slot order, with slot_pos = -1, which moe_combine skips; the
 * expert groups follow (offsets[0] = D, counts exclude them), so no group
 * holds a dropped row, and offsets[E] = T*k still. */
int moe_permute(const moe_shape* s, const int32_t* topk_idx, int32_t* counts,
                int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                void* stream);

/* moe_permute_capacity: moe_permute with an expert capacity: every expert
 * keeps at most `capacity` copies and drops the rest (yunthe page, section
 * 3.1, expert capacity; Baidu page, section 三.2, capacity-bound token
 * dropping).  Reading: an expert keeps its first `capacity` copies in slot
 * order s = t*k + j (earlier tokens first); a dropped copy adds nothing to
 * its token's output; the kept weights are not renormalised.
 *   capacity   >= 0 (MOE_ERR_INVALID_ARG otherwise); capacity >= T keeps
 *              every copy of a router's output (moe_permute's result)
 *   counts[e]  copies expert e keeps, min(copies of e, capacity)
 * Dropped rows [0, D): first the copies with ids outside [0, E) (slot
 * order), then the copies over capacity, by expert id, slot order inside
 * one expert; slot_pos = -1.  Kept rows: group e is offsets[e] ..
 * offsets[e+1], ascending slot; offsets[0] = D, offsets[E] = T*k. */
int moe_permute_capacity(const moe_shape* s, const int32_t* topk_idx,
                         int64_t capacity, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_slot, int32_t* slot_pos, void* stream);

/* Capacity from a capacity factor (yunthe page, sections 4.1 and 5.2: the
 * factor, typically 1.0 to 2.0, scales an expert's even share of the
 * copies): ceil(capacity_factor * T * k / E).  Host only, no HIP call.
 * Returns -1 for T < 0, k < 1, E < 1, a factor outside [0, 1e9] or a
 * capacity of 4e18 or more. */
int64_t moe_expert_capacity(int64_t T, int64_t k, int64_t E,
                            double capacity_factor);

/* ------------------------------------------------------------------ step 4
 * moe_grouped_gemm_gate_up: first expert GEMM with the SwiGLU epilogue.
 * For every row r of expert group e (offsets[e] <= r < offsets[e+1]):
 *   token t = sorted_slot[r] / k          (r <  T*k)
 *           = (r - T*k) % T               (shared rows)
 *   act[r, n] = silu(g) * u,  g = W_gate_up[e, n, :] . x[t, :],
 *                             u = W_gate_up[e, f + n, :] . x[t, :],
 *   silu(z) = z / (1 + exp(-z)), 0 <= n < f.
 *   W_gate_up [E+S, 2f, d] dt   act [R, f] dt out.
 * Experts with no rows are skipped (for T <= 64 each of their column tiles
 * may read one K step of weights, loaded before the row count is known). */
int moe_grouped_gemm_gate_up(const moe_shape* s, const void* x,
                             const int32_t* sorted_slot, const int32_t* offsets,
                             const void* W_gate_up, void* act, void* stream);

/* moe_grouped_gemm_down: second expert GEMM.
 *   expert_out[r, i] = W_down[e, i, :] . act[r, :] for the rows of group e.
 *   act [R, f] dt,  W_down [E+S, d, f] dt,  expert_out [R, d] dt out. */
int moe_grouped_gemm_down(const moe_shape* s, const void* act,
                          const int32_t* offsets, const void* W_down,
                          void* expert_out, void* stream);

/* moe_grouped_gemm: both expert GEMMs (gate_up + SwiGLU, then down). */
int moe_grouped_gemm(const moe_shape* s, const void* x,
                     const int32_t* sorted_slot, const int32_t* offsets,
                     const void* W_gate_up, const void* W_down, void* act,
                     void* expert_out, void* stream);

/* ------------------------------------------------------------------ step 5
 * moe_combine: weighted un-permute back to token order.
 *   y[t] = sum_{j<k} topk_w[t,j] * expert_out[slot_pos[t*k+j]]
 *        + sum_{sigma<S} expert_out[T*k + sigma*T + t]
 * accumulated in fp32 in that fixed order (no atomics), rounded to dt.
 * Copies with slot_pos < 0 (dropped by moe_permute) add nothing.
 *   expert_out [R, d] dt,  slot_pos [T*k],  topk_w [T, k],  y [T, d] dt out. */
int moe_combine(const moe_shape* s, const void* expert_out,
                const int32_t* slot_pos, const float* topk_w, void* y,
                void* stream);

/* ------------------------------------------------------------- whole layer
 * moe_layer_forward: steps 1-5 enqueued back to back on one stream (for bf16
 * batches of at most 64 tokens, the gate_up kernel finds each expert's rows
 * from the ids and writes the permutation itself: same results, one launch
 * fewer).
 * Intermediates live in the caller's workspace (device memory of at least
 * moe_workspace_size(s) bytes, 256-byte aligned); its layout is given by
 * moe_workspace_offsets.  y [T, d] dt out. */
size_t moe_workspace_size(const moe_shape* s);

enum {
  MOE_WS_TOPK_IDX = 0, /* int32 [T, k]     */
  MOE_WS_TOPK_W,       /* float [T, k]     */
  MOE_WS_COUNTS,       /* int32 [E+S]      */
  MOE_WS_OFFSETS,      /* int32 [E+S+1]    */
  MOE_WS_SORTED_SLOT,  /* int32 [T*k]      */
  MOE_WS_SLOT_POS,     /* int32 [T*k]      */
  MOE_WS_ACT,          /* dt    [R, f]     */
  MOE_WS_EXPERT_OUT,   /* dt    [R, d]     */
  MOE_WS_COUNT
};

/* Byte offsets of the intermediates inside the workspace; out has
 * MOE_WS_COUNT entries.  Returns MOE_OK or MOE_ERR_INVALID_ARG. */
int moe_workspace_offsets(const moe_shape* s, size_t* out);

int moe_layer_forward(const moe_shape* s, const void* x, const void* W_router,
                      const float* bias, const void* W_gate_up,
                      const void* W_down, void* y, void* workspace,
                      size_t workspace_bytes, void* stream);

/* moe_layer_forward_capacity: the layer with an expert capacity (step 3 is
 * moe_permute_capacity; dropped copies add nothing to y; shared experts are
 * not limited).  capacity >= 0; workspace as moe_layer_forward (same size
 * and layout). */
int moe_layer_forward_capacity(const moe_shape* s, const void* x,
                               const void* W_router, const float* bias,
                               const void* W_gate_up, const void* W_down,
                               int64_t capacity, void* y, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------- MXFP4 expert weights
 * The expert GEMMs and the whole layer with expert weights in MXFP4 (the
 * model-native quantisation that the aitoday "MoEs in Transformers" page,
 * section "From Dense to Sparse", expects faster kernels from; per-expert
 * quantisation in the packed layout: section "Dynamic Weight Loading with
 * WeightConverter").  Weight-only: x, act, expert_out, y and the router stay
 * bf16, so results are those of the bf16 entry points on the dequantised
 * weights (exact bf16 numbers).
 * Format (OCP Microscaling; the pages name it without defining it): FP4
 * E2M1 elements (bit 3 sign, bits 2-1 exponent e, bit 0 mantissa m: e = 0
 * gives m/2, else 2^(e-1)(1 + m/2)), two per byte with the even element in
 * the low nibble; one E8M0 scale byte X per 32 consecutive elements of a
 * weight row, factor 2^(X-127).  X = 255 (NaN in the format) is not
 * supported: the kernels read it as 2^128 and give inf or NaN.
 *   Wq_gate_up [E+S, 2f, d/2] uint8, Ws_gate_up [E+S, 2f, d/32] uint8
 *   Wq_down    [E+S, d, f/2]  uint8, Ws_down    [E+S, d, f/32]  uint8
 * (the packed bf16 layouts with each row's K elements packed).
 * Shapes: dt = MOE_DT_BF16, T <= 64 (decode batches), d and f multiples of
 * 32; others get MOE_ERR_UNSUPPORTED.  Weight tensors 16-byte aligned.
 * Experts without rows read none of their weights. */
int moe_grouped_gemm_gate_up_mxfp4(const moe_shape* s, const void* x,
                                   const int32_t* sorted_slot,
                                   const int32_t* offsets,
                                   const uint8_t* Wq_gate_up,
                                   const uint8_t* Ws_gate_up, void* act,
                                   void* stream);

int moe_grouped_gemm_down_mxfp4(const moe_shape* s, const void* act,
                                const int32_t* offsets, const uint8_t* Wq_down,
                                const uint8_t* Ws_down, void* expert_out,
                                void* stream);

/* Steps 1-5 with MXFP4 expert weights (route, permute, the two MXFP4
 * GEMMs, combine); workspace as moe_layer_forward (same size and layout). */
int moe_layer_forward_mxfp4(const moe_shape* s, const void* x,
                            const void* W_router, const float* bias,
                            const uint8_t* Wq_gate_up, const uint8_t* Ws_gate_up,
                            const uint8_t* Wq_down, const uint8_t* Ws_down,
                            void* y, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------- backward
 * moe_layer_backward: the gradients of a loss L with respect to the layer's
 * input and weights, given dL/dy (grouped-GEMM training: aitoday "MoEs in
 * Transformers" page, section "Training MoEs with Transformers").  The
 * chain rule through the forward above:
 *   dO = w dy_t per routed copy (dy_t per shared row), dw_tj = dy_t . O_tj,
 *   da = Wd_e^T dO, dg = da u silu'(g), du = da silu(g) with [g; u] = Wgu_e x_t
 *   (recomputed), dx_t = sum over its rows of Wgu_e^T [dg; du]
 *   + sum_j dl_tj Wr_{e_tj}, dWd_e = sum dO a^T, dWgu_e = sum [dg; du] x^T,
 *   dl_tj = w_tj (dw_tj - sum_i w_ti dw_ti) (softmax over the k selected
 *   logits), dWr_e = sum dl x, db_e = sum dl.
 * The selection of the k experts has no gradient; unselected experts get
 * zero gradients.
 *   x, W_router, W_gate_up, W_down  the forward's inputs (dt = MOE_DT_BF16
 *                only; MOE_ERR_UNSUPPORTED otherwise)
 *   dy           [T, d] bf16
 *   fwd_workspace the workspace of the moe_layer_forward (or
 *                moe_layer_forward_capacity) call on the same inputs: its
 *                routing, permutation, act and expert_out are used
 *   dx [T, d], dW_router [E, d], db [E], dW_gate_up [E+S, 2f, d],
 *   dW_down [E+S, d, f]: float32 out (every element written)
 *   dw           [T, k] float32 out (dL/d topk_w), or NULL
 *   workspace    moe_backward_workspace_size(s) bytes, 256-byte aligned
 * Intermediates dO and dH are bf16 (GEMM operands), everything else fp32;
 * sums in a fixed order (repeated calls are bitwise identical).  A copy
 * dropped by a capacity (slot_pos < 0) adds no expert gradient and gets
 * dw = 0; its weight still enters the softmax over the k selected logits
 * (the kept weights are not renormalised), so its logit's dl is
 * -w_tj sum_i w_ti dw_ti and reaches dx, dW_router and db. */
size_t moe_backward_workspace_size(const moe_shape* s);

int moe_layer_backward(const moe_shape* s, const void* x, const void* W_router,
                       const void* W_gate_up, const void* W_down, const void* dy,
                       const void* fwd_workspace, size_t fwd_workspace_bytes,
                       float* dx, float* dW_router, float* db, float* dW_gate_up,
                       float* dW_down, float* dw, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------- whole layer, no allocation
 * moe_layer_forward_static: moe_layer_forward with the intermediates in a
 * static device array of the library instead of a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  It allocates
 * nothing and frees nothing.
 *   - The array holds MOE_STATIC_SCRATCH_BYTES on every GPU the library
 *     runs on (on the calling thread's current device, which must be the
 *     stream's), from the library's load until the process ends.
 *   - Shapes whose moe_workspace_size exceeds it are rejected with
 *     MOE_ERR_WORKSPACE before any HIP call (e.g. decode batches fit;
 *     large prefill batches do not).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, or different threads) race and
 *     must be serialised by the caller.  Nothing in the array needs to start
 *     at zero; each call overwrites what it reads.
 * Arguments, results and errors are those of moe_layer_forward; the first
 * call on a device also looks up the array's address there (MOE_ERR_HIP if
 * that fails). */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)

int moe_layer_forward_static(const moe_shape* s, const void* x, const void* W_router,
                             const float* bias, const void* W_gate_up,
                             const void* W_down, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
