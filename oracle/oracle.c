/*
 * CPU oracle for the SageAttention-style quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline leg of the benchmark, never by the GPU library. Plain C, one step
 * at a time, in the order the method states them; built without fast-math and
 * with floating-point contraction off, so every float operation written here
 * is one correctly rounded IEEE operation.
 *
 * Where the pages (the SageAttention-RDNA4 v0.4.0 release notes and the
 * kernels-community issue "aiter-sage-attention") leave a step open, the
 * reading taken is stated at the step.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- BF16 --- */

float oracle_bf16_decode(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t oracle_bf16_encode(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040); /* stay a quiet NaN */
  uint32_t lower = u & 0xFFFFu, upper = u >> 16;
  /* round to nearest, ties to even, on the 16 discarded bits */
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1;
  return (uint16_t)upper;
}

/* ---------------------------------------------------------- FP8 (E4M3) --- */
/* OCP 8-bit floating point specification, E4M3: exponent bias 7, 3 stored
 * mantissa bits, exponent field 0 holds subnormals m * 2^-9, no infinities,
 * S.1111.111 is NaN, so the largest finite magnitude is 1.75 * 2^8 = 448. */

float oracle_e4m3_decode(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(sign ? -v : v);
}

/* Reading (the pages only say "FP8"): round to nearest with ties to the even
 * code; magnitudes above 448 saturate to 448 (the conversion's saturating
 * mode); the sign of zero is kept; NaN encodes as 0x7F. */
uint8_t oracle_e4m3_encode(float x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (a > 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {
    /* subnormal range: a / 2^-9 rounded to an integer 0..8; 8 is the
     * smallest normal 2^-6, whose code (exponent 1, mantissa 0) is also 8 */
    double m = nearbyint(ldexp(a, 9)); /* default mode: ties to even */
    return sign | (uint8_t)m;
  }
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  int ue = e - 1;          /* a = (2f) * 2^ue, 2f in [1, 2) */
  double m = nearbyint((2.0 * f - 1.0) * 8.0); /* exact scaling, then ties to even */
  if (m == 8.0) { m = 0.0; ue += 1; }
  int field = ue + 7;
  uint8_t code = (uint8_t)((field << 3) | (int)m);
  if (code > 0x7E) code = 0x7E; /* rounding up past 448 saturates */
  return sign | code;
}

/* ------------------------------------------------ INT8 block quantization */
/* Issue, "The kernel": Q and K are quantized per 32-row block. Reading: one
 * block is 32 consecutive tokens of one head times all D channels (a tail
 * block holds the remaining rows); symmetric absmax scaling onto [-127, 127]
 * with scale = a/127; codes are rint(x * (127/a)) (round half to even), so the
 * division happens once per block.
 * Blocks of tiny values: for a below 2^-64 the quotient 127/a can exceed the
 * largest float (it does below about 3.7e-37, which finite BF16 inputs and
 * mean-subtracted keys reach), so such a block is first multiplied by 2^64,
 * exactly for every element, and a with it; the codes are then formed as
 * above from the scaled values. Wherever 127/a is a finite float the codes are
 * the same as without the step: the scaled quotient is exactly 2^-64 times the
 * unscaled one and the scaled element exactly 2^64 times the unscaled one, so
 * every product rounds the same real number. The scale stays a/127 of the
 * unscaled a (it may be subnormal, or 0 below about 127 * 2^-150). */
#define ORACLE_TINY 0x1p-64f
#define ORACLE_TINY_LIFT 0x1p64f

float oracle_quant_block_int8(const float* x, int64_t rows, int64_t D, int8_t* q) {
  float a = 0.0f;
  for (int64_t i = 0; i < rows * D; ++i) {
    float ax = fabsf(x[i]);
    if (ax > a) a = ax;
  }
  if (a == 0.0f) {
    memset(q, 0, (size_t)(rows * D));
    return 0.0f;
  }
  float scale = a / 127.0f;
  float lift = a < ORACLE_TINY ? ORACLE_TINY_LIFT : 1.0f;
  float inv = 127.0f / (a * lift);
  for (int64_t i = 0; i < rows * D; ++i) {
    float y = (x[i] * lift) * inv;
    float r = rintf(y);
    if (r > 127.0f) r = 127.0f;
    /* for finite inputs r is finite; the comparison is written so that a NaN
     * (possible only from non-finite inputs, outside the method's domain)
     * still gives a defined integer conversion */
    if (!(r >= -127.0f)) r = -127.0f;
    q[i] = (int8_t)r;
  }
  return scale;
}

/* ---------------------------------------------------------- fp64 sum --- */
/* Release notes, "What changed": with smooth_k on, the key mean is summed in
 * fp64. Reading: the fp64 sum of a channel is its exact sum rounded once to
 * double (nearest, ties to even), the most accurate fp64 sum and the same in
 * whatever order the terms are taken.
 * A finite BF16 value is M * 2^(e - 133) with an integer 0 <= M < 256 and
 * 0 <= e <= 253 (exponent field E > 0: M = 128 + mantissa, e = E - 1; E = 0:
 * M = mantissa, e = 0), so the exact sum of n < 2^25 of them is an integer
 * multiple of 2^-133 below 2^286 in magnitude. It is accumulated here as two
 * non-negative integers (positive and negative terms) of ten 32-bit limbs,
 * then rounded. Returns NaN if a value is not finite. */
#define ORACLE_LIMBS 10

static void big_add_shifted(uint32_t* acc, uint32_t M, int e) {
  uint64_t carry = (uint64_t)M << (e % 32);   /* < 2^39, spans limbs e/32 and e/32 + 1 */
  for (int j = e / 32; j < ORACLE_LIMBS && carry != 0; ++j) {
    uint64_t t = (uint64_t)acc[j] + (carry & 0xFFFFFFFFu);
    acc[j] = (uint32_t)t;
    carry = (carry >> 32) + (t >> 32);
  }
}

static int big_bit(const uint32_t* x, int bit) { return (int)((x[bit / 32] >> (bit % 32)) & 1u); }

double oracle_bf16_exact_sum(const uint16_t* x, int64_t n, int64_t stride) {
  uint32_t pos[ORACLE_LIMBS] = {0}, neg[ORACLE_LIMBS] = {0};
  for (int64_t i = 0; i < n; ++i) {
    uint16_t b = x[i * stride];
    uint32_t E = (b >> 7) & 0xFFu, man = b & 0x7Fu;
    if (E == 0xFFu) return NAN;
    uint32_t M = E ? 128u + man : man;
    int e = E ? (int)E - 1 : 0;
    big_add_shifted((b >> 15) ? neg : pos, M, e);
  }
  /* magnitude = |pos - neg|, by limbs from the most significant */
  int negative = 0;
  for (int j = ORACLE_LIMBS - 1; j >= 0; --j)
    if (pos[j] != neg[j]) { negative = neg[j] > pos[j]; break; }
  const uint32_t* big = negative ? neg : pos;
  const uint32_t* small = negative ? pos : neg;
  uint32_t mag[ORACLE_LIMBS];
  int64_t borrow = 0;
  for (int j = 0; j < ORACLE_LIMBS; ++j) {
    int64_t t = (int64_t)big[j] - (int64_t)small[j] - borrow;
    borrow = t < 0;
    mag[j] = (uint32_t)(t + (borrow ? ((int64_t)1 << 32) : 0));
  }
  /* most significant set bit */
  int p = 32 * ORACLE_LIMBS - 1;
  while (p >= 0 && !big_bit(mag, p)) --p;
  if (p < 0) return 0.0;
  /* the top 64 bits (or all of them), with every lower bit ORed into bit 0:
   * bit 0 lies below the rounding position of a 53-bit significand, so the
   * one rounding of the uint64 -> double conversion is the rounding of the
   * whole magnitude */
  uint64_t u = 0;
  int low = p >= 63 ? p - 63 : 0;
  for (int bit = p; bit >= low; --bit) u = (u << 1) | (uint64_t)big_bit(mag, bit);
  int sticky = 0;
  for (int bit = low - 1; bit >= 0; --bit) sticky |= big_bit(mag, bit);
  u |= (uint64_t)sticky;
  double d = ldexp((double)u, low - 133);
  return negative ? -d : d;
}

/* ----------------------------------------------------------- prologue --- */
int oracle_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S, int64_t D,
                        int64_t row_stride, int smooth_k, int64_t S_pad, int8_t* q8, float* q_scale, int8_t* k8,
                        float* k_scale, uint8_t* v8t, float* v_scale, float* k_mean) {
  if (S < 0 || D < 1 || S_pad < S) return -1;
  int64_t nb = (S + 31) / 32;
  float* rowsbuf = (float*)malloc((size_t)(32 * D) * sizeof(float));
  if (!rowsbuf) return -1;

  /* Release notes, "What changed": with smooth_k on, the key mean is summed
   * in fp64. Reading: per channel d, the exact sum over all S tokens rounded
   * once to double (oracle_bf16_exact_sum), divided by S in double, rounded
   * once to float; it is then subtracted from every key in float. With
   * smooth_k off nothing is subtracted and k_mean is zero. */
  for (int64_t d = 0; d < D; ++d) {
    float km = 0.0f;
    if (smooth_k && S > 0) km = (float)(oracle_bf16_exact_sum(k + d, S, row_stride) / (double)S);
    k_mean[d] = km;
  }

  for (int64_t n = 0; n < nb; ++n) {
    int64_t r0 = 32 * n, rows = (S - r0 < 32) ? S - r0 : 32;
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t d = 0; d < D; ++d) rowsbuf[r * D + d] = oracle_bf16_decode(q[(r0 + r) * row_stride + d]);
    q_scale[n] = oracle_quant_block_int8(rowsbuf, rows, D, q8 + r0 * D);

    for (int64_t r = 0; r < rows; ++r)
      for (int64_t d = 0; d < D; ++d) {
        float x = oracle_bf16_decode(k[(r0 + r) * row_stride + d]);
        rowsbuf[r * D + d] = smooth_k ? x - k_mean[d] : x;
      }
    k_scale[n] = oracle_quant_block_int8(rowsbuf, rows, D, k8 + r0 * D);
  }

  /* Issue, "The kernel": V is quantized per channel. Reading: FP8 E4M3 with
   * absmax scaling onto [-448, 448] per channel over the whole sequence,
   * scale = a/448, codes e4m3(v * (448/a)); stored transposed (channel-major,
   * keys contiguous) and zero-padded to S_pad keys. */
  for (int64_t d = 0; d < D; ++d) {
    float a = 0.0f;
    for (int64_t s = 0; s < S; ++s) {
      float ax = fabsf(oracle_bf16_decode(v[s * row_stride + d]));
      if (ax > a) a = ax;
    }
    uint8_t* dst = v8t + d * S_pad;
    if (a == 0.0f) {
      v_scale[d] = 0.0f;
      memset(dst, 0, (size_t)S_pad);
      continue;
    }
    v_scale[d] = a / 448.0f;
    /* a channel of tiny values is lifted by 2^64 first, as an INT8 block is
     * (448/a overflows below about 1.3e-36); the codes are unchanged wherever
     * 448/a is a finite float */
    float lift = a < ORACLE_TINY ? ORACLE_TINY_LIFT : 1.0f;
    float inv = 448.0f / (a * lift);
    for (int64_t s = 0; s < S; ++s)
      dst[s] = oracle_e4m3_encode((oracle_bf16_decode(v[s * row_stride + d]) * lift) * inv);
    for (int64_t s = S; s < S_pad; ++s) dst[s] = 0;
  }
  free(rowsbuf);
  return 0;
}

/* ---------------------------------------------------------- attention --- */
/* Issue, "The kernel": QK^T in INT8 and PV in FP8, both accumulated in FP32.
 * Readings for the steps the pages leave open:
 *   - score t_ij = float(sum_d q8[i,d]*k8[j,d]) * c_ij with
 *     c_ij = (q_scale[i/32] * k_scale[j/32]) * (sm_scale * log2(e)), all in
 *     float (log2(e) rounded to float), so that exp2(t) = exp(q.k*sm_scale);
 *   - online softmax over key tiles of T keys in ascending order starting at
 *     key 0 (the last tile may be short): m' = max(m, max_tile t),
 *     alpha = exp2(m - m') (0 for the first tile), p_j = exp2(t_j - m'),
 *     l = alpha*l + sum_tile p_j;
 *   - P requantized as e4m3(448 * p_j) (p_j <= 1, so the static scale 448
 *     uses the whole FP8 range), PV accumulated in float as
 *     o_d = alpha*o_d + sum_tile dec(p8_j) * dec(v8[j,d]);
 *   - output bf16((o_d * v_scale[d]) / (448 * l)).
 * Sums inside a tile run in ascending key order.
 * Causal (an extension: the pages reject it): query i sees keys 0 .. i only,
 * i.e. the row is computed exactly as above over the first i + 1 keys, with
 * the same tiles from key 0 (the last one cut at key i). */
int oracle_attn_rows(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                     const uint8_t* v8t, int64_t S_pad, const float* v_scale, int64_t S, int64_t D, float sm_scale,
                     int64_t T, int causal, const int64_t* rows, int64_t nrows, float* out_f32, uint16_t* out_bf16,
                     float* lse_out) {
  if (S < 1 || D < 1 || T < 1 || S_pad < S) return -1;
  const float log2e = 1.44269504088896340736f;
  const float sl2 = sm_scale * log2e;
  float* t = (float*)malloc((size_t)T * sizeof(float));
  float* pdec = (float*)malloc((size_t)T * sizeof(float));
  float* o = (float*)malloc((size_t)D * sizeof(float));
  if (!t || !pdec || !o) { free(t); free(pdec); free(o); return -1; }

  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows[r];
    if (i < 0 || i >= S) { free(t); free(pdec); free(o); return -1; }
    const int8_t* qi = q8 + i * D;
    float qs = q_scale[i / 32];
    float m = -INFINITY, l = 0.0f;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0f;

    const int64_t nk = causal ? i + 1 : S;   /* keys this row sees */
    for (int64_t j0 = 0; j0 < nk; j0 += T) {
      int64_t n = (nk - j0 < T) ? nk - j0 : T;
      float tmax = -INFINITY;
      for (int64_t jj = 0; jj < n; ++jj) {
        int64_t j = j0 + jj;
        const int8_t* kj = k8 + j * D;
        int32_t acc = 0;
        for (int64_t d = 0; d < D; ++d) acc += (int32_t)qi[d] * (int32_t)kj[d];
        float c = (qs * k_scale[j / 32]) * sl2;
        t[jj] = (float)acc * c;
        if (t[jj] > tmax) tmax = t[jj];
      }
      float mnew = m > tmax ? m : tmax;
      float alpha = exp2f(m - mnew); /* m = -inf on the first tile gives 0 */
      float psum = 0.0f;
      for (int64_t jj = 0; jj < n; ++jj) {
        float p = exp2f(t[jj] - mnew);
        psum += p;
        pdec[jj] = oracle_e4m3_decode(oracle_e4m3_encode(448.0f * p));
      }
      l = alpha * l + psum;
      for (int64_t d = 0; d < D; ++d) {
        const uint8_t* vd = v8t + d * S_pad + j0;
        float acc = 0.0f;
        for (int64_t jj = 0; jj < n; ++jj) acc += pdec[jj] * oracle_e4m3_decode(vd[jj]);
        o[d] = alpha * o[d] + acc;
      }
      m = mnew;
    }
    /* log-sum-exp of the dequantized scores s_j = t_j ln 2: after the last
     * tile, l = sum_j 2^(t_j - m), so ln sum_j e^(s_j) = m ln 2 + ln l. */
    if (lse_out) lse_out[r] = (float)((double)m * 0.69314718055994530942 + log((double)l));
    float denom = 448.0f * l;
    for (int64_t d = 0; d < D; ++d) {
      float val = (o[d] * v_scale[d]) / denom;
      if (out_f32) out_f32[r * D + d] = val;
      if (out_bf16) out_bf16[r * D + d] = oracle_bf16_encode(val);
    }
  }
  free(t); free(pdec); free(o);
  return 0;
}

/* Exact attention in double: softmax(q k^T * sm_scale) v, the quantity the
 * method approximates (no quantization, no tiling); causal: keys j <= i. */
int oracle_exact_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S, int64_t D,
                      int64_t row_stride, double sm_scale, int causal, const int64_t* rows, int64_t nrows,
                      double* out, double* lse_out) {
  if (S < 1 || D < 1) return -1;
  double* s = (double*)malloc((size_t)S * sizeof(double));
  if (!s) return -1;
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t i = rows[r];
    if (i < 0 || i >= S) { free(s); return -1; }
    const int64_t nk = causal ? i + 1 : S;   /* keys j <= i when causal */
    double mx = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d)
        acc += (double)oracle_bf16_decode(q[i * row_stride + d]) * (double)oracle_bf16_decode(k[j * row_stride + d]);
      s[j] = acc * sm_scale;
      if (s[j] > mx) mx = s[j];
    }
    double den = 0.0;
    for (int64_t j = 0; j < nk; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
    if (lse_out) lse_out[r] = mx + log(den);   /* ln sum_j e^(s_j) */
    for (int64_t d = 0; d < D; ++d) {
      double num = 0.0;
      for (int64_t j = 0; j < nk; ++j) num += s[j] * (double)oracle_bf16_decode(v[j * row_stride + d]);
      out[r * D + d] = num / den;
    }
  }
  free(s);
  return 0;
}
