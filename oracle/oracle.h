/*
 * CPU oracle for the SageAttention-style quantized attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The GPU library never
 * includes, links or calls it, and it shares no code with the GPU path.
 *
 * Sources (the pages: the "SageAttention-RDNA4 v0.4.0" release notes, and the
 * kernels-community issue "aiter-sage-attention: SageAttention for AMD RDNA4
 * (gfx1201)"):
 *   - issue, section "The kernel": QK^T runs in INT8 and PV in FP8, both with
 *     FP32 accumulation; Q and K are quantized per 32-row block and V per
 *     channel.
 *   - release notes, "What changed", fourth item: with smooth_k on, the key
 *     mean is summed in fp64 (read as the exact sum rounded once to double).
 *   - issue, "What I have so far": the accepted problem is BF16 [B,S,H,128],
 *     equal Q/K/V shapes, no mask, non-causal.
 * Steps the pages leave open (absmax scaling, e4m3 for V, the exp2 online
 * softmax, FP8 requantization of P, rounding modes, the key-tile schedule)
 * follow one written reading each; every function below states its reading.
 *
 * All functions are single-threaded and work on one head (b,h) at a time;
 * callers parallelise over heads or rows. Arrays are dense, row-major.
 */
#ifndef SAGE_ORACLE_H
#define SAGE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* BF16 <-> float. Decoding is exact; encoding rounds to nearest, ties to even. */
float oracle_bf16_decode(uint16_t b);
uint16_t oracle_bf16_encode(float f);

/* OCP 8-bit floating point, E4M3 flavour (bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 is NaN, largest finite 448). Encoding rounds to the
 * nearest finite value with ties to the even code, saturates magnitudes above
 * 448 to +-448, keeps the sign of zero, and maps NaN to 0x7F. */
uint8_t oracle_e4m3_encode(float x);
float oracle_e4m3_decode(uint8_t c);

/* INT8 quantization of one 32-row block (rows x D floats, rows <= 32):
 * a = max|x|; scale = a/127; q = rint(x * (127/a)) clamped to [-127,127]
 * (each a single correctly rounded float operation; ties to even).
 * A block with a < 2^-64 is multiplied by 2^64 first (x and a), which keeps
 * 127/a finite and changes no code wherever it was finite already.
 * An all-zero block gets scale 0 and all-zero codes. Returns the scale. */
float oracle_quant_block_int8(const float* x, int64_t rows, int64_t D, int8_t* q);

/* Exact sum of n BF16 values x[0], x[stride], ... rounded once to double
 * (nearest, ties to even): the reading of "summed in fp64". NaN if a value
 * is not finite. */
double oracle_bf16_exact_sum(const uint16_t* x, int64_t n, int64_t stride);

/* The prologue for one head. q, k, v point at row s=0 of the head in a BF16
 * tensor whose consecutive rows (tokens) are row_stride elements apart (H*D
 * for the [B,S,H,D] layout). D elements of a row are contiguous.
 * Outputs (nb = ceil(S/32), S_pad >= S):
 *   q8[S][D], q_scale[nb], k8[S][D], k_scale[nb]   INT8 per 32-row block
 *   v8t[D][S_pad], v_scale[D]                      e4m3 per channel, transposed,
 *                                                  columns S..S_pad-1 zero (a
 *                                                  channel with absmax < 2^-64
 *                                                  is lifted by 2^64 first, as
 *                                                  an INT8 block is)
 *   k_mean[D]                                      smooth_k: float of (the exact
 *                                                  sum rounded to double) / S;
 *                                                  else zeros
 * Inputs must be finite, and with smooth_k every K - k_mean must be a finite
 * float (true whenever |K| <= 2^126); other inputs give unspecified codes.
 * Returns 0, or -1 for S < 0 or D < 1. */
int oracle_prepare_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S, int64_t D,
                        int64_t row_stride, int smooth_k, int64_t S_pad, int8_t* q8, float* q_scale, int8_t* k8,
                        float* k_scale, uint8_t* v8t, float* v_scale, float* k_mean);

/* Quantized attention for selected query rows of one head, from the prologue's
 * outputs: INT8 scores, dequantization by q_scale*k_scale*sm_scale (with
 * log2(e) folded in for exp2), online softmax in float over key tiles of T
 * keys taken in ascending order from key 0, P requantized to e4m3 as
 * e4m3(448*p), PV accumulated in float, BF16 output.
 * out_f32[n][D] receives the float value before BF16 rounding (may be NULL);
 * out_bf16[n][D] the BF16 result; lse_out[n] (may be NULL) the natural-log
 * sum of exponentials of the row's dequantized scores, m ln 2 + ln l from the
 * final running maximum m (log2 units) and l = sum_j 2^(t_j - m), evaluated
 * in double and rounded once to float. causal != 0: row i sees keys 0 .. i
 * only (same tiles from key 0). Returns 0, or -1 for bad arguments. */
int oracle_attn_rows(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                     const uint8_t* v8t, int64_t S_pad, const float* v_scale, int64_t S, int64_t D, float sm_scale,
                     int64_t T, int causal, const int64_t* rows, int64_t nrows, float* out_f32, uint16_t* out_bf16,
                     float* lse_out);

/* Exact softmax(q k^T * sm_scale) v in double for selected rows of one head,
 * from the unquantized BF16 inputs (same addressing as oracle_prepare_head);
 * lse_out[n] (may be NULL) receives ln sum_j exp(q.k_j * sm_scale). */
int oracle_exact_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S, int64_t D,
                      int64_t row_stride, double sm_scale, int causal, const int64_t* rows, int64_t nrows,
                      double* out, double* lse_out);

#ifdef __cplusplus
}
#endif
#endif
