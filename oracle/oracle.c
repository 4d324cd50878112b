/*
 * oracle.c -- plain fp64 CPU definition of one sparse-routed MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  It is written for
 * a reader to check against the pages by eye: one token at a time, serial
 * fp64 sums in ascending index order, no blocking, no fusion, no reordering.
 * The only parallelism is an OpenMP loop over independent tokens or rows,
 * which does not change any sum.
 *
 * Citations (page title, section): see oracle.h for the list of readings.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Widen element i of a dt-typed buffer to fp64.  bfloat16 is the upper half
 * of a binary32 pattern, so widening it is a 16-bit left shift. */
static double elem(const void* p, int dt, int64_t i) {
  if (dt == ORACLE_F32) return (double)((const float*)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float v;
  memcpy(&v, &bits, sizeof v);
  return (double)v;
}

/* Dot product of row `row` of a [rows, n] dt-typed matrix with an fp64
 * vector, summed serially in ascending index order. */
static double dot_row(const void* M, int dt, int64_t row, int64_t n,
                      const double* v) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += elem(M, dt, row * n + i) * v[i];
  return s;
}

static int bad_dt(int dt) { return dt != ORACLE_F32 && dt != ORACLE_BF16; }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---------------------------------------------------------------- routing */

/* Expert order for top-k: larger logit first; equal logits, lower index
 * first (the tie rule).  qsort with this total order is deterministic. */
typedef struct {
  double logit;
  int32_t e;
} ranked;

static int by_logit_then_index(const void* pa, const void* pb) {
  const ranked* a = (const ranked*)pa;
  const ranked* b = (const ranked*)pb;
  if (a->logit > b->logit) return -1;
  if (a->logit < b->logit) return 1;
  return (a->e > b->e) - (a->e < b->e);
}

/* Route one token: logits (score of every expert from the router linear
 * layer), softmax over all experts, the k experts with the largest logits,
 * and their probabilities renormalised over the k selected ones.
 * If forced != NULL the selection is those k experts instead.
 * scratch holds E doubles (logits) and E ranked entries. */
static void route_token(int64_t t, int64_t d, int64_t E, int64_t k, int dt,
                        const void* x, const void* W_router, const float* bias,
                        const int32_t* forced, double* xt, double* logit,
                        ranked* order, int32_t* idx, double* w) {
  for (int64_t i = 0; i < d; ++i) xt[i] = elem(x, dt, t * d + i);

  /* 1. logits: l_e = sum_i x[t,i] W_router[e,i]  (+ b_e) */
  for (int64_t e = 0; e < E; ++e) {
    logit[e] = dot_row(W_router, dt, e, d, xt);
    if (bias) logit[e] += (double)bias[e];
  }

  /* 2. softmax over all experts: p_e = exp(l_e - max) / sum_e exp(l_e - max) */
  double m = logit[0];
  for (int64_t e = 1; e < E; ++e)
    if (logit[e] > m) m = logit[e];
  double z = 0.0;
  for (int64_t e = 0; e < E; ++e) z += exp(logit[e] - m);

  /* 3. top-k by logit, ties to the lower index */
  if (forced) {
    for (int64_t j = 0; j < k; ++j) idx[j] = forced[j];
  } else {
    for (int64_t e = 0; e < E; ++e) {
      order[e].logit = logit[e];
      order[e].e = (int32_t)e;
    }
    qsort(order, (size_t)E, sizeof(ranked), by_logit_then_index);
    for (int64_t j = 0; j < k; ++j) idx[j] = order[j].e;
  }

  /* 4. renormalise the selected probabilities so they sum to one */
  double sel = 0.0;
  for (int64_t j = 0; j < k; ++j) sel += exp(logit[idx[j]] - m) / z;
  for (int64_t j = 0; j < k; ++j) w[j] = (exp(logit[idx[j]] - m) / z) / sel;
}

int oracle_route(int64_t T, int64_t d, int64_t E, int64_t k, int dt,
                 const void* x, const void* W_router, const float* bias,
                 double* logits, int32_t* idx, double* w) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E || bad_dt(dt)) return -1;
  if (!x || !W_router || !idx || !w) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    ranked* order = (ranked*)malloc(sizeof(ranked) * (size_t)E);
    if (!xt || !lg || !order) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < T; ++t) {
        route_token(t, d, E, k, dt, x, W_router, bias, NULL, xt, lg, order,
                    idx + t * k, w + t * k);
        if (logits) memcpy(logits + t * E, lg, sizeof(double) * (size_t)E);
      }
    }
    free(xt);
    free(lg);
    free(order);
  }
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------ permutation */

/* Counting-sort permutation of the T*k token copies by expert id, with an
 * optional expert capacity (capacity < 0: none).
 *
 * Expert capacity: every expert accepts at most `capacity` token copies and
 * the overflow is dropped (yunthe "分工的艺术" page, section 3.1, expert
 * capacity; Baidu page, section 三.2, capacity-constrained token dropping;
 * yunthe page, sections 4.1 and 5.2, capacity factor).  Readings: an expert
 * keeps its first `capacity` copies in slot order s = t*k + j (earlier
 * tokens first); a dropped copy adds nothing to its token's output and the
 * kept weights are not renormalised.
 *
 * Row layout of the permuted buffers:
 *   rows [0, D)        the D dropped copies, by expert id, ascending slot
 *                      inside one expert; their slot_pos is -1;
 *   rows offsets[e] .. offsets[e] + counts[e]
 *                      the copies expert e keeps, ascending slot;
 *                      counts[e] = min(copies of e, capacity);
 *   offsets[0] = D, offsets[E] = T*k; shared expert sigma: T rows from
 *   T*k + sigma*T, token order. */
int oracle_permute_capacity(int64_t T, int64_t k, int64_t E, int64_t S,
                            int64_t capacity, const int32_t* idx,
                            int32_t* counts, int32_t* offsets,
                            int32_t* sorted_slot, int32_t* slot_pos) {
  if (T < 0 || k < 1 || E < 1 || S < 0) return -1;
  if (!counts || !offsets || (T > 0 && (!idx || !sorted_slot || !slot_pos)))
    return -1;
  int64_t n = T * k;
  for (int64_t s = 0; s < n; ++s)
    if (idx[s] < 0 || idx[s] >= E) return -1;
  int64_t cap = capacity < 0 || capacity > n ? n : capacity;

  /* copies per expert, then what each keeps and drops */
  int64_t* total = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* drop_base = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* seen = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  if (!total || !drop_base || !seen) {
    free(total);
    free(drop_base);
    free(seen);
    return -2;
  }
  for (int64_t s = 0; s < n; ++s) total[idx[s]] += 1;
  int64_t dropped = 0;
  for (int64_t e = 0; e < E; ++e) {
    int64_t kept = total[e] < cap ? total[e] : cap;
    counts[e] = (int32_t)kept;
    drop_base[e] = dropped;
    dropped += total[e] - kept;
  }
  /* every shared expert takes all T tokens */
  for (int64_t sg = 0; sg < S; ++sg) counts[E + sg] = (int32_t)T;

  /* exclusive prefix sum of the kept counts, after the dropped rows */
  offsets[0] = (int32_t)dropped;
  for (int64_t e = 0; e < E + S; ++e) offsets[e + 1] = offsets[e] + counts[e];

  /* stable scatter: slots visited in ascending order */
  for (int64_t s = 0; s < n; ++s) {
    int32_t e = idx[s];
    int64_t r = seen[e]++; /* earlier copies of expert e */
    int64_t pos;
    if (r < cap) {
      pos = offsets[e] + r;
      slot_pos[s] = (int32_t)pos;
    } else {
      pos = drop_base[e] + (r - cap);
      slot_pos[s] = -1;
    }
    sorted_slot[pos] = (int32_t)s;
  }
  free(total);
  free(drop_base);
  free(seen);
  return 0;
}

int oracle_permute(int64_t T, int64_t k, int64_t E, int64_t S,
                   const int32_t* idx, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_slot, int32_t* slot_pos) {
  return oracle_permute_capacity(T, k, E, S, -1, idx, counts, offsets,
                                 sorted_slot, slot_pos);
}

int64_t oracle_expert_capacity(int64_t T, int64_t k, int64_t E,
                               double factor) {
  /* capacity factor times the even share T*k/E of one expert, rounded up */
  if (T < 0 || k < 1 || E < 1 || !(factor >= 0.0)) return -1;
  return (int64_t)ceil(factor * (double)(T * k) / (double)E);
}

/* -------------------------------------------------------- balance loss */

/* Load-balance statistics of the router (yunthe page, section 3.1, the load
 * balance loss example; the gate it averages is the softmax over all experts
 * of that page's section 1.1 gating code):
 *   probs[t, e]    = softmax over the E experts of token t's logits
 *                    (logits as in routing, bias included);
 *   importance[e]  = mean over the T tokens of probs[t, e]
 *                    (T = 0: 0/0, NaN);
 *   loss           = KL divergence of the uniform target u = 1/E from
 *                    log(importance + 1e-8), batch-mean reduced over the
 *                    E-long input, i.e.
 *                    (1/E) * sum_e u * (log u - log(importance[e] + 1e-8)).
 * probs ([T, E]) is optional. */
int oracle_balance(int64_t T, int64_t d, int64_t E, int dt, const void* x,
                   const void* W_router, const float* bias, double* probs,
                   double* importance, double* loss) {
  if (T < 0 || d < 1 || E < 1 || bad_dt(dt)) return -1;
  if (!importance || !loss || (T > 0 && (!x || !W_router))) return -1;
  double* P = probs;
  if (!P && T > 0) {
    P = (double*)malloc(sizeof(double) * (size_t)(T * E));
    if (!P) return -2;
  }
  int fail = 0;
#pragma omp parallel
  {
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    if (!xt) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < T; ++t) {
        double* pt = P + t * E;
        for (int64_t i = 0; i < d; ++i) xt[i] = elem(x, dt, t * d + i);
        for (int64_t e = 0; e < E; ++e) {
          pt[e] = dot_row(W_router, dt, e, d, xt);
          if (bias) pt[e] += (double)bias[e];
        }
        double m = pt[0];
        for (int64_t e = 1; e < E; ++e)
          if (pt[e] > m) m = pt[e];
        double z = 0.0;
        for (int64_t e = 0; e < E; ++e) z += exp(pt[e] - m);
        for (int64_t e = 0; e < E; ++e) pt[e] = exp(pt[e] - m) / z;
      }
    }
    free(xt);
  }
  if (!fail) {
    /* mean over tokens, summed in token order */
    for (int64_t e = 0; e < E; ++e) {
      double s = 0.0;
      for (int64_t t = 0; t < T; ++t) s += P[t * E + e];
      importance[e] = s / (double)T;
    }
    double u = 1.0 / (double)E;
    double kl = 0.0;
    for (int64_t e = 0; e < E; ++e)
      kl += u * (log(u) - log(importance[e] + 1e-8));
    *loss = kl / (double)E;
  }
  if (P != probs) free(P);
  return fail ? -2 : 0;
}

/* ------------------------------------------------------------ expert FFN */

/* SwiGLU hidden activation of token vector xt through expert e:
 * gate = rows [0, f) of the packed gate_up matrix (w1), up = rows [f, 2f)
 * (w3); a_n = silu(gate_n) * up_n. */
static void expert_hidden(int64_t e, int64_t d, int64_t f, int dt,
                          const void* W_gate_up, const double* xt,
                          double* act) {
  int64_t base = e * 2 * f; /* first row of expert e in [E+S, 2f, d] */
  for (int64_t n = 0; n < f; ++n) {
    double g = dot_row(W_gate_up, dt, base + n, d, xt);
    double u = dot_row(W_gate_up, dt, base + f + n, d, xt);
    double silu = g / (1.0 + exp(-g));
    act[n] = silu * u;
  }
}

/* Down projection of activation vector act through expert e:
 * out_i = sum_n W_down[e, i, n] act_n. */
static void expert_down(int64_t e, int64_t d, int64_t f, int dt,
                        const void* W_down, const double* act, double* out) {
  for (int64_t i = 0; i < d; ++i)
    out[i] = dot_row(W_down, dt, e * d + i, f, act);
}

int oracle_gate_up_rows(int64_t n, const int64_t* tok, const int32_t* expert,
                        int64_t d, int64_t f, int dt, const void* x,
                        const void* W_gate_up, double* act) {
  if (n < 0 || d < 1 || f < 1 || bad_dt(dt)) return -1;
  if (n > 0 && (!tok || !expert || !x || !W_gate_up || !act)) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    if (!xt) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < d; ++i) xt[i] = elem(x, dt, tok[r] * d + i);
        expert_hidden(expert[r], d, f, dt, W_gate_up, xt, act + r * f);
      }
    }
    free(xt);
  }
  return fail ? -2 : 0;
}

int oracle_down_rows(int64_t n, const int32_t* expert, int64_t d, int64_t f,
                     int dt, const void* act, const void* W_down, double* out) {
  if (n < 0 || d < 1 || f < 1 || bad_dt(dt)) return -1;
  if (n > 0 && (!expert || !act || !W_down || !out)) return -1;
  int fail = 0;
#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)f);
    if (!a) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < n; ++r) {
        for (int64_t i = 0; i < f; ++i) a[i] = elem(act, dt, r * f + i);
        expert_down(expert[r], d, f, dt, W_down, a, out + r * d);
      }
    }
    free(a);
  }
  return fail ? -2 : 0;
}

/* ------------------------------------------------------- MXFP4 weights */

/* One FP4 (E2M1) element: bit 3 sign, bits 2-1 exponent e, bit 0 mantissa
 * m; e = 0 encodes m * 1/2 (subnormal), otherwise 2^(e-1) * (1 + m/2). */
static double e2m1_value(unsigned code) {
  unsigned e = (code >> 1) & 3u, m = code & 1u;
  double mag = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

/* Dequantise an MXFP4 matrix [rows, K] (the OCP Microscaling format that
 * the aitoday page names as the model's native quantisation, section "From
 * Dense to Sparse"; its layout is the OCP specification's, which the pages
 * do not give): each run of 32 consecutive elements of a row shares one
 * E8M0 scale byte X, value 2^(X - 127) (X = 255: NaN); elements are FP4
 * E2M1, two per byte, element 2i in the low nibble of byte i.
 * q: [rows, K/2] bytes, scales: [rows, K/32] bytes, out: [rows, K] fp64. */
int oracle_dequant_mxfp4(int64_t rows, int64_t K, const uint8_t* q,
                         const uint8_t* scales, double* out) {
  if (rows < 0 || K < 0 || K % 32 != 0) return -1;
  if (rows > 0 && K > 0 && (!q || !scales || !out)) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < K; ++i) {
      uint8_t byte = q[r * (K / 2) + i / 2];
      unsigned code = (i % 2 == 0) ? (byte & 15u) : (byte >> 4);
      uint8_t x = scales[r * (K / 32) + i / 32];
      double scale = x == 255 ? NAN : ldexp(1.0, (int)x - 127);
      out[r * K + i] = e2m1_value(code) * scale;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- combine */

int oracle_combine(int64_t T, int64_t k, int64_t S, int64_t d, int dt,
                   const void* O, const int32_t* slot_pos, const double* w,
                   double* y) {
  if (T < 0 || k < 1 || S < 0 || d < 1 || bad_dt(dt)) return -1;
  if (T > 0 && (!O || !slot_pos || !w || !y)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < k; ++j) {
        int64_t row = slot_pos[t * k + j];
        if (row < 0) continue; /* a copy dropped by a capacity adds nothing */
        acc += w[t * k + j] * elem(O, dt, row * d + i);
      }
      for (int64_t sg = 0; sg < S; ++sg) {
        int64_t row = T * k + sg * T + t;
        acc += elem(O, dt, row * d + i);
      }
      y[t * d + i] = acc;
    }
  }
  return 0;
}

/* With an expert capacity, whether a copy is kept depends on the copies of
 * every earlier token: route all tokens first, then walk the copies in slot
 * order, each expert keeping its first `capacity` (the reading of
 * oracle_permute_capacity).  *keep_out: [T*k], 1 = kept; the caller frees. */
static int capacity_keep(int64_t T, int64_t d, int64_t E, int64_t k, int dt, const void* x,
                         const void* W_router, const float* bias, int64_t capacity,
                         uint8_t** keep_out) {
  int32_t* idx_all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k));
  double* w_all = (double*)malloc(sizeof(double) * (size_t)(T * k));
  int64_t* seen = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  uint8_t* keep = (uint8_t*)malloc((size_t)(T * k));
  int rc = (idx_all && w_all && seen && keep) ? 0 : -2;
  if (rc == 0) rc = oracle_route(T, d, E, k, dt, x, W_router, bias, NULL, idx_all, w_all);
  if (rc == 0)
    for (int64_t s = 0; s < T * k; ++s) keep[s] = seen[idx_all[s]]++ < capacity;
  free(idx_all);
  free(w_all);
  free(seen);
  if (rc != 0) {
    free(keep);
    keep = NULL;
  }
  *keep_out = keep;
  return rc;
}

/* ------------------------------------------------------------ whole layer */

int oracle_layer_forward(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                         int64_t S, int dt, const void* x, const void* W_router,
                         const float* bias, const void* W_gate_up,
                         const void* W_down, int64_t n_tok,
                         const int64_t* tok_list, const int32_t* forced_idx,
                         int64_t capacity, int32_t* idx_out, double* w_out,
                         double* y) {
  if (T < 0 || d < 1 || f < 1 || E < 1 || k < 1 || k > E || S < 0 ||
      bad_dt(dt))
    return -1;
  if (capacity >= 0 && forced_idx) return -1;
  if (!tok_list) n_tok = T;
  if (n_tok < 0) return -1;
  if (n_tok > 0 && (!x || !W_router || !W_gate_up || !W_down || !y)) return -1;
  if (tok_list)
    for (int64_t q = 0; q < n_tok; ++q)
      if (tok_list[q] < 0 || tok_list[q] >= T) return -1;
  if (forced_idx)
    for (int64_t q = 0; q < n_tok * k; ++q)
      if (forced_idx[q] < 0 || forced_idx[q] >= E) return -1;

  uint8_t* keep = NULL;
  if (capacity >= 0 && T > 0) {
    int rc = capacity_keep(T, d, E, k, dt, x, W_router, bias, capacity, &keep);
    if (rc != 0) return rc;
  }

  int fail = 0;
#pragma omp parallel
  {
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    double* lg = (double*)malloc(sizeof(double) * (size_t)E);
    ranked* order = (ranked*)malloc(sizeof(ranked) * (size_t)E);
    double* act = (double*)malloc(sizeof(double) * (size_t)f);
    double* out = (double*)malloc(sizeof(double) * (size_t)d);
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    if (!xt || !lg || !order || !act || !out || !idx || !w) {
#pragma omp atomic write
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t q = 0; q < n_tok; ++q) {
        int64_t t = tok_list ? tok_list[q] : q;
        route_token(t, d, E, k, dt, x, W_router, bias,
                    forced_idx ? forced_idx + q * k : NULL, xt, lg, order, idx,
                    w);
        /* route_token leaves x[t] widened in xt */
        double* yt = y + q * d;
        for (int64_t i = 0; i < d; ++i) yt[i] = 0.0;
        /* y_t = sum_j w_j Expert_{idx_j}(x_t): selected experts only (and
         * of those, the copies their expert keeps) */
        for (int64_t j = 0; j < k; ++j) {
          if (keep && !keep[t * k + j]) continue;
          expert_hidden(idx[j], d, f, dt, W_gate_up, xt, act);
          expert_down(idx[j], d, f, dt, W_down, act, out);
          for (int64_t i = 0; i < d; ++i) yt[i] += w[j] * out[i];
        }
        /* + every shared expert with weight one */
        for (int64_t sg = 0; sg < S; ++sg) {
          expert_hidden(E + sg, d, f, dt, W_gate_up, xt, act);
          expert_down(E + sg, d, f, dt, W_down, act, out);
          for (int64_t i = 0; i < d; ++i) yt[i] += out[i];
        }
        if (idx_out) memcpy(idx_out + q * k, idx, sizeof(int32_t) * (size_t)k);
        if (w_out) memcpy(w_out + q * k, w, sizeof(double) * (size_t)k);
      }
    }
    free(xt);
    free(lg);
    free(order);
    free(act);
    free(out);
    free(idx);
    free(w);
  }
  free(keep);
  return fail ? -2 : 0;
}

/* --------------------------------------------------------------- backward */

/* Gradients of the layer, the backward pass that grouped-GEMM training runs
 * (aitoday "MoEs in Transformers" page, section "Training MoEs with
 * Transformers").  They are the derivatives of the forward defined above
 * by the chain rule, for a loss whose gradient with respect to y is dy:
 *   y_t = sum_j w_tj O_tj + sum_s O_ts,   O = Wd_e a,   a = silu(g) * u,
 *   [g; u] = Wgu_e x_t,   w_tj = exp(l_tj) / sum_{i<k} exp(l_ti),
 *   l_te = Wr_e . x_t + b_e;
 *   dO_tj = w_tj dy_t (shared experts: dy_t),  dw_tj = dy_t . O_tj,
 *   da = Wd_e^T dO,  dg = da * u * silu'(g),  du = da * silu(g),
 *   silu'(g) = s (1 + g (1 - s)) with s = 1 / (1 + e^-g),
 *   dx_t += Wgu_e^T [dg; du],  dWd_e += dO a^T,  dWgu_e += [dg; du] x_t^T,
 *   dl_tj = w_tj (dw_tj - sum_i w_ti dw_ti)   (softmax over the k selected),
 *   dx_t += sum_j dl_tj Wr_{e_tj},  dWr_e += dl x_t,  db_e += dl.
 * The choice of the k experts is piecewise constant in the logits: it has
 * no gradient, and unselected experts get none.
 * Outputs (fp64, each optional):
 *   dx [n_tok, d] for the listed tokens (tok_list NULL: all T);
 *   dWgu [n_exp, 2f, d] and dWd [n_exp, d, f] for the listed experts
 *   (indices 0 .. E+S-1; shared experts after the routed ones);
 *   dWr [E, d], db [E], dw [T, k].
 * Tokens are visited in order and every sum is serial, in ascending index
 * order (experts in slot order, then the shared ones, then the router). */
int oracle_layer_backward(int64_t T, int64_t d, int64_t f, int64_t E, int64_t k,
                          int64_t S, int dt, const void* x, const void* W_router,
                          const float* bias, const void* W_gate_up,
                          const void* W_down, const void* dy, int64_t capacity, int64_t n_tok,
                          const int64_t* tok_list, double* dx, int64_t n_exp,
                          const int32_t* exp_list, double* dWgu, double* dWd,
                          double* dWr, double* db, double* dw) {
  if (T < 0 || d < 1 || f < 1 || E < 1 || k < 1 || k > E || S < 0 || bad_dt(dt))
    return -1;
  if (!tok_list) n_tok = T;
  if (n_tok < 0 || n_exp < 0) return -1;
  if (T > 0 && (!x || !W_router || !W_gate_up || !W_down || !dy)) return -1;
  if (n_tok > 0 && !dx) return -1;
  if (n_exp > 0 && (!exp_list || !dWgu || !dWd)) return -1;
  int64_t G = E + S;
  int64_t* tok_pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
  int64_t* exp_pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)G);
  double* xt = (double*)malloc(sizeof(double) * (size_t)d);
  double* lg = (double*)malloc(sizeof(double) * (size_t)E);
  ranked* order = (ranked*)malloc(sizeof(ranked) * (size_t)E);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* w = (double*)malloc(sizeof(double) * (size_t)k);
  double* dwt = (double*)malloc(sizeof(double) * (size_t)k);
  double* g = (double*)malloc(sizeof(double) * (size_t)f);
  double* u = (double*)malloc(sizeof(double) * (size_t)f);
  double* a = (double*)malloc(sizeof(double) * (size_t)f);
  double* da = (double*)malloc(sizeof(double) * (size_t)f);
  double* dg = (double*)malloc(sizeof(double) * (size_t)f);
  double* du = (double*)malloc(sizeof(double) * (size_t)f);
  double* O = (double*)malloc(sizeof(double) * (size_t)d);
  double* dO = (double*)malloc(sizeof(double) * (size_t)d);
  double* dxt = (double*)malloc(sizeof(double) * (size_t)d);
  uint8_t* keep = NULL; /* [T*k] kept copies, with a capacity only */
  int rc = 0;
  if (!tok_pos || !exp_pos || !xt || !lg || !order || !idx || !w || !dwt || !g || !u ||
      !a || !da || !dg || !du || !O || !dO || !dxt) {
    rc = -2;
    goto done;
  }
  for (int64_t t = 0; t < T; ++t) tok_pos[t] = -1;
  for (int64_t q = 0; q < n_tok; ++q) {
    int64_t t = tok_list ? tok_list[q] : q;
    if (t < 0 || t >= T || tok_pos[t] >= 0) {
      rc = -1;
      goto done;
    }
    tok_pos[t] = q;
  }
  for (int64_t e = 0; e < G; ++e) exp_pos[e] = -1;
  for (int64_t q = 0; q < n_exp; ++q) {
    if (exp_list[q] < 0 || exp_list[q] >= G || exp_pos[exp_list[q]] >= 0) {
      rc = -1;
      goto done;
    }
    exp_pos[exp_list[q]] = q;
  }
  if (n_tok > 0) memset(dx, 0, sizeof(double) * (size_t)(n_tok * d));
  if (n_exp > 0) {
    memset(dWgu, 0, sizeof(double) * (size_t)(n_exp * 2 * f * d));
    memset(dWd, 0, sizeof(double) * (size_t)(n_exp * d * f));
  }
  if (dWr) memset(dWr, 0, sizeof(double) * (size_t)(E * d));
  if (db) memset(db, 0, sizeof(double) * (size_t)E);
  int router_grads = dWr || db || dw;
  /* copies dropped by an expert capacity add nothing to y: no expert
   * gradient, and dw = 0 (their weights still enter the softmax of the k
   * selected logits, so dl keeps its form) */
  if (capacity >= 0 && T > 0) {
    rc = capacity_keep(T, d, E, k, dt, x, W_router, bias, capacity, &keep);
    if (rc != 0) goto done;
  }

  for (int64_t t = 0; t < T; ++t) {
    int listed = tok_pos[t] >= 0;
    if (!listed && n_exp == 0 && !router_grads) continue;
    route_token(t, d, E, k, dt, x, W_router, bias, NULL, xt, lg, order, idx, w);
    for (int64_t c = 0; c < d; ++c) dxt[c] = 0.0;
    for (int64_t j = 0; j < k + S; ++j) {
      int routed = j < k;
      int64_t e = routed ? idx[j] : E + (j - k);
      double wj = routed ? w[j] : 1.0;
      if (routed && keep && !keep[t * k + j]) {
        dwt[j] = 0.0;
        continue;
      }
      int want_e = exp_pos[e] >= 0;
      int need_O = routed && (listed || router_grads);
      if (!listed && !want_e && !need_O) continue;
      /* forward through expert e: [g; u] = Wgu_e x_t, a = silu(g) * u */
      int64_t base = 2 * f * e; /* first gate_up row of expert e */
      for (int64_t n = 0; n < f; ++n) {
        g[n] = dot_row(W_gate_up, dt, base + n, d, xt);
        u[n] = dot_row(W_gate_up, dt, base + f + n, d, xt);
        a[n] = g[n] / (1.0 + exp(-g[n])) * u[n];
      }
      if (need_O) {
        /* dw_tj = dy_t . O_tj */
        double acc = 0.0;
        for (int64_t i = 0; i < d; ++i) {
          O[i] = dot_row(W_down, dt, e * d + i, f, a);
          acc += elem(dy, dt, t * d + i) * O[i];
        }
        dwt[j] = acc;
      }
      if (!listed && !want_e) continue;
      /* dO = w dy_t; da = Wd_e^T dO; SwiGLU backward */
      for (int64_t i = 0; i < d; ++i) dO[i] = wj * elem(dy, dt, t * d + i);
      for (int64_t n = 0; n < f; ++n) {
        double acc = 0.0;
        for (int64_t i = 0; i < d; ++i) acc += elem(W_down, dt, (e * d + i) * f + n) * dO[i];
        da[n] = acc;
        double sg = 1.0 / (1.0 + exp(-g[n]));
        dg[n] = da[n] * u[n] * (sg * (1.0 + g[n] * (1.0 - sg)));
        du[n] = da[n] * (g[n] * sg);
      }
      if (listed) {
        /* dx_t += Wgu_e^T [dg; du] */
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t n = 0; n < f; ++n) {
            acc += elem(W_gate_up, dt, (base + n) * d + c) * dg[n];
            acc += elem(W_gate_up, dt, (base + f + n) * d + c) * du[n];
          }
          dxt[c] += acc;
        }
      }
      if (want_e) {
        double* gd = dWd + exp_pos[e] * d * f;
        double* gu = dWgu + exp_pos[e] * 2 * f * d;
        for (int64_t i = 0; i < d; ++i)
          for (int64_t n = 0; n < f; ++n) gd[i * f + n] += dO[i] * a[n];
        for (int64_t n = 0; n < f; ++n)
          for (int64_t c = 0; c < d; ++c) {
            gu[n * d + c] += dg[n] * xt[c];
            gu[(f + n) * d + c] += du[n] * xt[c];
          }
      }
    }
    if (listed || router_grads) {
      /* softmax over the k selected logits: dl_j = w_j (dw_j - sum_i w_i dw_i) */
      double sw = 0.0;
      for (int64_t j = 0; j < k; ++j) sw += w[j] * dwt[j];
      for (int64_t j = 0; j < k; ++j) {
        double dl = w[j] * (dwt[j] - sw);
        int64_t e = idx[j];
        if (listed)
          for (int64_t c = 0; c < d; ++c) dxt[c] += dl * elem(W_router, dt, e * d + c);
        if (dWr)
          for (int64_t c = 0; c < d; ++c) dWr[e * d + c] += dl * xt[c];
        if (db) db[e] += dl;
        if (dw) dw[t * k + j] = dwt[j];
      }
    }
    if (listed) memcpy(dx + tok_pos[t] * d, dxt, sizeof(double) * (size_t)d);
  }
done:
  free(keep);
  free(tok_pos);
  free(exp_pos);
  free(xt);
  free(lg);
  free(order);
  free(idx);
  free(w);
  free(dwt);
  free(g);
  free(u);
  free(a);
  free(da);
  free(dg);
  free(du);
  free(O);
  free(dO);
  free(dxt);
  return rc;
}
