/* Runs every oracle function on small inputs, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (test infrastructure, like the oracle):
 * any out-of-bounds access, leak or undefined operation aborts the run.
 * Inputs come from a fixed linear congruential generator. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static unsigned long long g_state = 12345;
static float uniform(void) { /* in [-1, 1) */
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (float)((g_state >> 40) & 0xffffff) / 8388608.0f - 1.0f;
}
static float* floats(size_t n, float scale) {
  float* a = (float*)malloc(sizeof(float) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) a[i] = uniform() * scale;
  return a;
}

int main(void) {
  int fails = 0;
  const int64_t T = 9, d = 16, f = 8, E = 5, k = 2, S = 1, G = E + S;
  float* x = floats(T * d, 1.0f);
  float* Wr = floats(E * d, 0.5f);
  float* Wgu = floats(G * 2 * f * d, 0.3f);
  float* Wd = floats(G * d * f, 0.3f);
  float* dy = floats(T * d, 1.0f);
  float bias[5] = {0.1f, -0.2f, 0.3f, 0.0f, -0.5f};
  double* logits = (double*)malloc(sizeof(double) * T * E);
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * T * k);
  double* w = (double*)malloc(sizeof(double) * T * k);
  fails += oracle_route(T, d, E, k, ORACLE_F32, x, Wr, bias, logits, idx, w) != 0;
  int32_t counts[6], offsets[7], ss[18], sp[18];
  fails += oracle_permute(T, k, E, S, idx, counts, offsets, ss, sp) != 0;
  for (int64_t cap = 0; cap < 4; ++cap)
    fails += oracle_permute_capacity(T, k, E, S, cap, idx, counts, offsets, ss, sp) != 0;
  fails += oracle_permute(0, k, E, S, NULL, counts, offsets, NULL, NULL) != 0;
  fails += oracle_expert_capacity(T, k, E, 1.5) != 6; /* ceil(1.5 * 18 / 5) */
  double imp[5], loss, probs[45];
  fails += oracle_balance(T, d, E, ORACLE_F32, x, Wr, bias, probs, imp, &loss) != 0;
  fails += oracle_balance(0, d, E, ORACLE_F32, NULL, Wr, NULL, NULL, imp, &loss) != 0;
  int64_t toks[3] = {0, 4, 8};
  int64_t tok_all[18];
  int32_t ex_all[18];
  for (int64_t r = 0; r < T * k; ++r) {
    tok_all[r] = ss[r] / k;
    ex_all[r] = idx[ss[r]];
  }
  double* act = (double*)malloc(sizeof(double) * T * k * f);
  fails += oracle_gate_up_rows(T * k, tok_all, ex_all, d, f, ORACLE_F32, x, Wgu, act) != 0;
  float* act32 = (float*)malloc(sizeof(float) * T * k * f);
  for (int64_t i = 0; i < T * k * f; ++i) act32[i] = (float)act[i];
  double* O = (double*)malloc(sizeof(double) * T * k * d);
  fails += oracle_down_rows(T * k, ex_all, d, f, ORACLE_F32, act32, Wd, O) != 0;
  float* O32 = (float*)malloc(sizeof(float) * (T * k + S * T) * d);
  memset(O32, 0, sizeof(float) * (T * k + S * T) * d);
  double* yc = (double*)malloc(sizeof(double) * T * d);
  /* slot_pos of the last capacity permutation holds dropped copies (-1) */
  fails += oracle_combine(T, k, S, d, ORACLE_F32, O32, sp, w, yc) != 0;
  fails += oracle_permute(T, k, E, S, idx, counts, offsets, ss, sp) != 0;
  fails += oracle_combine(T, k, S, d, ORACLE_F32, O32, sp, w, yc) != 0;
  double* y = (double*)malloc(sizeof(double) * T * d);
  fails += oracle_layer_forward(T, d, f, E, k, S, ORACLE_F32, x, Wr, bias, Wgu, Wd, 3, toks,
                                NULL, -1, idx, w, y) != 0;
  fails += oracle_layer_forward(T, d, f, E, k, S, ORACLE_F32, x, Wr, bias, Wgu, Wd, 0, NULL,
                                NULL, 2, NULL, NULL, y) != 0;
  int32_t forced[6] = {4, 3, 0, 1, 2, 4};
  fails += oracle_layer_forward(T, d, f, E, k, S, ORACLE_F32, x, Wr, bias, Wgu, Wd, 3, toks,
                                forced, -1, NULL, NULL, y) != 0;
  unsigned char q[2 * 16], sc[2];
  for (int i = 0; i < 32; ++i) q[i] = (unsigned char)(i * 37);
  sc[0] = 127;
  sc[1] = 255;
  double dq[64];
  fails += oracle_dequant_mxfp4(2, 32, q, sc, dq) != 0;
  fails += !isnan(dq[40]);
  double* dx = (double*)malloc(sizeof(double) * 3 * d);
  double* dWgu = (double*)malloc(sizeof(double) * G * 2 * f * d);
  double* dWd = (double*)malloc(sizeof(double) * G * d * f);
  double* dWr = (double*)malloc(sizeof(double) * E * d);
  double db[5], dw[18];
  int32_t exps[6] = {0, 1, 2, 3, 4, 5};
  fails += oracle_layer_backward(T, d, f, E, k, S, ORACLE_F32, x, Wr, bias, Wgu, Wd, dy, 2, 3,
                                 toks, dx, G, exps, dWgu, dWd, dWr, db, dw) != 0;
  /* rejected arguments */
  fails += oracle_route(T, d, E, E + 1, ORACLE_F32, x, Wr, NULL, NULL, idx, w) == 0;
  fails += oracle_dequant_mxfp4(1, 31, q, sc, dq) == 0;
  int64_t dup[2] = {1, 1};
  fails += oracle_layer_backward(T, d, f, E, k, S, ORACLE_F32, x, Wr, bias, Wgu, Wd, dy, -1, 2,
                                 dup, dx, 0, NULL, NULL, NULL, NULL, NULL, NULL) == 0;
  free(x); free(Wr); free(Wgu); free(Wd); free(dy); free(logits); free(idx); free(w);
  free(act); free(act32); free(O); free(O32); free(yc); free(y); free(dx); free(dWgu);
  free(dWd); free(dWr);
  printf("%s: %d failures\n", fails ? "FAIL" : "ok", fails);
  return fails ? 1 : 0;
}
