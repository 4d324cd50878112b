/*
 * oracle.h -- plain fp64 CPU definition of one sparse-routed MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this library: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; the two meet only in the seeded input buffers.
 *
 * What is computed, and where the pages define it:
 *   - Router score per expert from a small linear layer, then softmax and
 *     top-k (Baidu "MoE稀疏架构是什么" page, section 三.1 and the section 四
 *     pseudocode; yunthe "分工的艺术" page, section 1.1 gating code; qqiyuan
 *     2026 MoE guide, the MoELayer pseudocode).
 *   - The selected weights renormalised to sum to one (Baidu page, section 四:
 *     softmax taken over the top-k scores, which equals softmax-over-all then
 *     renormalise over the selected experts).
 *   - Token copies grouped by expert id (sort, then one grouped GEMM) and the
 *     results gathered back to token order (aitoday "MoEs in Transformers"
 *     page, section "Expert Backend", the grouped_mm backend).
 *   - Packed expert tensors: gate_up_proj = experts stacked on dim 0 with w1
 *     rows then w3 rows on dim 1, giving [E, 2f, d]; down_proj stacked on dim 0,
 *     giving [E, d, f] (aitoday page, section "Dynamic Weight Loading with
 *     WeightConverter").
 *   - Output = weighted sum of the selected experts' outputs only (Baidu page,
 *     section 四).
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes):
 *   - expert function: SwiGLU, a = silu(gate) * up, silu(z) = z / (1 + e^-z),
 *     then the down projection; no biases, no clamping, no scaling;
 *   - ranking key: the fp64 logit, ties to the lower expert index; slot j of a
 *     token holds its rank-j expert;
 *   - optional router bias b[E] (fp32) added to the logits before softmax;
 *   - shared experts: S extra experts stored after the E routed ones in both
 *     weight tensors, weight 1 for every token, outside the softmax;
 *   - permutation order inside one expert group: ascending slot id
 *     s = t*k + j (stable counting sort); shared groups follow the routed ones
 *     with rows T*k + sigma*T + t;
 *   - expert capacity (optional): an expert keeps its first `capacity`
 *     copies in slot order, dropped copies add nothing, kept weights are not
 *     renormalised;
 *   - balance loss: the gate averaged over tokens is the dense softmax over
 *     all experts (bias included).
 *
 * Element types: dt = ORACLE_F32 (IEEE binary32) or ORACLE_BF16 (bfloat16,
 * passed as its raw 16-bit pattern).  Every value is widened to fp64 before
 * use and every sum is a serial fp64 sum in ascending index order.
 *
 * All pointers are host pointers owned by the caller.  Functions return 0 on
 * success and a negative value for an invalid argument; nothing is allocated
 * that outlives a call.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

/* Routing of every token: fp64 logits[T,E] (optional, may be NULL), the top-k
 * expert ids idx[T,k] in rank order and their renormalised weights w[T,k]. */
int oracle_route(int64_t T, int64_t d, int64_t E, int64_t k, int dt,
                 const void* x, const void* W_router, const float* bias,
                 double* logits, int32_t* idx, double* w);

/* Counting-sort permutation of the T*k token copies by expert id.
 * counts[E+S], offsets[E+S+1], sorted_slot[T*k], slot_pos[T*k]. */
int oracle_permute(int64_t T, int64_t k, int64_t E, int64_t S,
                   const int32_t* idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_slot, int32_t* slot_pos);

/* The same with an expert capacity (capacity < 0: none): every expert keeps
 * its first `capacity` copies in slot order, the rest are dropped.  Rows
 * [0, D) of the permutation hold the D dropped copies (by expert id, then
 * slot) with slot_pos = -1; kept copies follow, offsets[0] = D,
 * offsets[E] = T*k, counts[e] = copies kept by expert e. */
int oracle_permute_capacity(int64_t T, int64_t k, int64_t E, int64_t S,
                            int64_t capacity, const int32_t* idx,
                            int32_t* counts, int32_t* offsets,
                            int32_t* sorted_slot, int32_t* slot_pos);

/* Capacity from a capacity factor: ceil(factor * T*k / E); -1 if invalid. */
int64_t oracle_expert_capacity(int64_t T, int64_t k, int64_t E, double factor);

/* Router load statistics: probs[T,E] (optional) = softmax over all experts
 * of each token's logits, importance[E] = its mean over tokens, and the
 * KL-to-uniform balance loss (1/E) sum_e (1/E)(log(1/E) - log(imp_e + 1e-8)). */
int oracle_balance(int64_t T, int64_t d, int64_t E, int dt, const void* x,
                   const void* W_router, const float* bias, double* probs,
                   double* importance, double* loss);

/* SwiGLU hidden activation of n (token, expert) pairs:
 * act[r, :] = silu(Wgu[e, 0:f, :] x[t]) * (Wgu[e, f:2f, :] x[t]),
 * with t = tok[r], e = expert[r].  act is [n, f] fp64. */
int oracle_gate_up_rows(int64_t n, const int64_t* tok, const int32_t* expert,
                        int64_t d, int64_t f, int dt, const void* x,
                        const void* W_gate_up, double* act);

/* Down projection of n given activation rows (element type dt, [n, f]):
 * out[r, :] = W_down[expert[r]] act[r].  out is [n, d] fp64. */
int oracle_down_rows(int64_t n, const int32_t* expert, int64_t d, int64_t f,
                     int dt, const void* act, const void* W_down, double* out);

/* MXFP4 weights (OCP Microscaling, FP4 E2M1 elements, one E8M0 scale per
 * 32 consecutive elements of a row, element 2i in the low nibble of byte
 * i): dequantise q [rows, K/2] with scales [rows, K/32] into out [rows, K]
 * fp64.  K must be a multiple of 32. */
int oracle_dequant_mxfp4(int64_t rows, int64_t K, const uint8_t* q,
                         const uint8_t* scales, double* out);

/* Weighted combine of expert-output rows stored in permuted order
 * (element type dt, [T*k + S*T, d]):
 * y[t] = sum_j w[t,j] * O[slot_pos[t*k+j]] + sum_sigma O[T*k + sigma*T + t];
 * copies with slot_pos < 0 (dropped by a capacity) add nothing. */
int oracle_combine(int64_t T, int64_t k, int64_t S, int64_t d, int dt,
                   const void* O, const int32_t* slot_pos, const double* w,
                   double* y);

/* The whole layer for n_tok listed tokens (tok_list == NULL: all T tokens, in
 * order).  y is [n_tok, d] fp64; idx_out / w_out ([n_tok, k], optional) get
 * the routing.  forced_idx ([n_tok, k], optional) replaces the selection by
 * the given expert ids; their weights are then the softmax over the given
 * experts' logits.  capacity >= 0 applies an expert capacity (as in
 * oracle_permute_capacity; dropped copies add nothing); it cannot be
 * combined with forced_idx. */
int oracle_layer_forward(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                         int64_t S, int dt, const void* x, const void* W_router,
                         const float* bias, const void* W_gate_up,
                         const void* W_down, int64_t n_tok,
                         const int64_t* tok_list, const int32_t* forced_idx,
                         int64_t capacity, int32_t* idx_out, double* w_out,
                         double* y);

/* Backward pass: gradients of sum(y * dy) (dy [T, d], element type dt) with
 * respect to x (listed tokens; tok_list NULL: all T), the listed experts'
 * gate_up and down weights (exp_list, indices 0 .. E+S-1), the router
 * weights and bias, and the routing weights (dw [T, k]); all fp64, each
 * optional.  dx [n_tok, d], dWgu [n_exp, 2f, d], dWd [n_exp, d, f],
 * dWr [E, d], db [E].  capacity >= 0: the forward with that expert capacity
 * (as oracle_layer_forward); dropped copies get no expert gradient and
 * dw = 0. */
int oracle_layer_backward(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                          int64_t S, int dt, const void* x, const void* W_router,
                          const float* bias, const void* W_gate_up,
                          const void* W_down, const void* dy, int64_t capacity, int64_t n_tok,
                          const int64_t* tok_list, double* dx, int64_t n_exp,
                          const int32_t* exp_list, double* dWgu, double* dWd,
                          double* dWr, double* db, double* dw);

/* Number of OpenMP threads the oracle uses (for reporting). */
int oracle_num_threads(void);
/* Threads of the following calls' parallel loops (n > 0), for timing. */
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
