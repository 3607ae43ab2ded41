/* Drives every oracle entry point on small seeded inputs (ragged lengths,
 * smooth_k on and off, causal and not, with and without the log-sum-exp, head
 * dims 64 and 128) for a build with AddressSanitizer and UndefinedBehavior-
 * Sanitizer. Exit status 0 means every call returned 0 and every output value
 * is finite; a sanitizer report aborts with a non-zero status. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double next_uniform(void) {   /* xorshift64*, test data only */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}

static uint16_t bf16_of(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

/* tiny = 1: Q, K and V values of order 1e-39 (BF16 subnormals, blocks and
 * channels whose absmax makes 127/a and 448/a overflow a float);
 * tiny = 2: K channels mixing magnitudes 2^60 and 2^-60 (an fp64 running sum
 * of them is not exact). */
static int run(int64_t S, int64_t D, int smooth_k, int tiny) {
  const int64_t S_pad = (S + 127) / 128 * 128, nb = (S + 31) / 32;
  uint16_t* q = malloc((size_t)(S * D) * 2);
  uint16_t* k = malloc((size_t)(S * D) * 2);
  uint16_t* v = malloc((size_t)(S * D) * 2);
  int8_t* q8 = malloc((size_t)(S * D));
  int8_t* k8 = malloc((size_t)(S * D));
  uint8_t* v8t = malloc((size_t)(D * S_pad));
  float* qs = malloc((size_t)nb * 4);
  float* ks = malloc((size_t)nb * 4);
  float* vs = malloc((size_t)D * 4);
  float* km = malloc((size_t)D * 4);
  const float f = tiny == 1 ? 1e-39f : 1.0f;
  for (int64_t i = 0; i < S * D; ++i) {
    q[i] = bf16_of((float)(4.0 * next_uniform() - 2.0) * f);
    k[i] = bf16_of((float)(3.0 * next_uniform() - 1.0) * f);
    v[i] = bf16_of((float)(2.0 * next_uniform() - 1.0) * f);
    if (tiny == 2) k[i] = bf16_of((float)(next_uniform() - 0.5) * ((i / D) % 2 ? 0x1p60f : 0x1p-60f));
  }
  int bad = oracle_prepare_head(q, k, v, S, D, D, smooth_k, S_pad, q8, qs, k8, ks, v8t, vs, km) != 0;
  int64_t rows[6] = {0, S / 3, S / 2, S - 1, S > 1 ? 1 : 0, S > 129 ? 128 : 0};
  float* of = malloc((size_t)(6 * D) * 4);
  uint16_t* ob = malloc((size_t)(6 * D) * 2);
  float* lse = malloc(6 * 4);
  double* oe = malloc((size_t)(6 * D) * 8);
  double* lse_e = malloc(6 * 8);
  for (int causal = 0; causal < 2 && !bad; ++causal) {
    bad |= oracle_attn_rows(q8, qs, k8, ks, v8t, S_pad, vs, S, D, 0.088f, 128, causal, rows, 6, of, ob, lse) != 0;
    bad |= oracle_attn_rows(q8, qs, k8, ks, v8t, S_pad, vs, S, D, 0.088f, 16, causal, rows, 6, NULL, ob, NULL) != 0;
    bad |= oracle_exact_rows(q, k, v, S, D, D, 0.088, causal, rows, 6, oe, lse_e) != 0;
    for (int i = 0; i < 6 * (int)D; ++i) bad |= !isfinite(of[i]) || !isfinite(oe[i]);
    /* the log-sum-exp of scores that all vanish is still finite; exact
     * attention's may underflow to ln 0 only in the tiny case */
    for (int i = 0; i < 6; ++i) bad |= !isfinite(lse[i]) || (!tiny && !isfinite(lse_e[i]));
  }
  free(q); free(k); free(v); free(q8); free(k8); free(v8t); free(qs); free(ks); free(vs); free(km);
  free(of); free(ob); free(lse); free(oe); free(lse_e);
  return bad;
}

int main(void) {
  const int64_t lengths[] = {1, 2, 31, 33, 128, 129, 300};
  int bad = 0;
  for (size_t i = 0; i < sizeof lengths / sizeof lengths[0]; ++i)
    for (int64_t D = 64; D <= 128; D += 64)
      for (int smooth = 0; smooth < 2; ++smooth)
        for (int tiny = 0; tiny < 3; ++tiny) {
          int r = run(lengths[i], D, smooth, tiny);
          if (r)
            fprintf(stderr, "failed: S=%lld D=%lld smooth_k=%d tiny=%d\n", (long long)lengths[i], (long long)D,
                    smooth, tiny);
          bad |= r;
        }
  /* the exact sum of a channel: 2^60, 1, -2^60 in that order sums to 1 */
  {
    const uint16_t x[3] = {bf16_of(0x1p60f), bf16_of(1.0f), bf16_of(-0x1p60f)};
    bad |= oracle_bf16_exact_sum(x, 3, 1) != 1.0;
  }
  /* argument checks: rows out of range, bad sizes */
  int64_t row = 5;
  bad |= oracle_attn_rows(NULL, NULL, NULL, NULL, NULL, 128, NULL, 4, 128, 0.1f, 128, 0, &row, 1, NULL, NULL, NULL) != -1;
  bad |= oracle_exact_rows(NULL, NULL, NULL, 0, 128, 128, 0.1, 0, &row, 1, NULL, NULL) != -1;
  printf(bad ? "FAIL\n" : "ok\n");
  return bad;
}
