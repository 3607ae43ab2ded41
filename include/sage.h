/*
 * sage.h - C ABI of the MI355X (gfx950) quantized attention forward.
 *
 * What it computes (the pages: the kernels-community issue "aiter-sage-attention:
 * SageAttention for AMD RDNA4 (gfx1201)", sections "The kernel" and "What I
 * have so far", and the "SageAttention-RDNA4 v0.4.0" release notes, "What
 * changed"):
 *   - a prologue quantizes Q and K to INT8 per 32-row block and V to FP8 per
 *     channel; with smooth_k the per-channel key mean, summed in fp64, is
 *     subtracted from K first;
 *   - the attention step computes QK^T in INT8 and PV in FP8, both with FP32
 *     accumulation, and writes BF16;
 *   - accepted inputs are BF16 [B, S, H, 128] with equal Q/K/V shapes and no
 *     mask; anything else is rejected with an error, never silently handled
 *     another way.
 * Extensions beyond the pages (whose package rejects them): head dim 64
 * (the layouts below then hold 64 where they say 128), the per-row
 * log-sum-exp output, and causal attention (query i sees keys 0 .. i).
 *
 * Conventions for every call:
 *   - All calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream of the current device). Device pointers must belong to
 *     the current device.
 *   - The caller owns every buffer. The library never allocates, frees or
 *     synchronises, and keeps no state between calls.
 *   - Validation is done on the host before any device call, in this order:
 *       1. null pointers, negative sizes, a tensor whose element count
 *          overflows 64 bits, non-finite or non-positive sm_scale
 *          -> SAGE_ERR_INVALID_ARGUMENT;
 *       2. dtype other than BF16, D not 64 or 128, unequal shapes,
 *          stride[3] != 1, a base address / row stride that is not 16-byte
 *          aligned, strides reaching past 2^60 elements, S > 2^25 - 128
 *          (33,554,304 tokens), or B * H * ceil(S / 128) >= 2^31 (the
 *          workgroup count of a launch) -> SAGE_ERR_UNSUPPORTED;
 *       3. workspace smaller than the *_workspace_bytes() figure
 *          -> SAGE_ERR_WORKSPACE_TOO_SMALL;
 *       4. current device is not gfx950 (or there is none) -> SAGE_ERR_UNSUPPORTED;
 *       5. a launch failure -> SAGE_ERR_DEVICE.
 *     sage_last_error() then returns a thread-local message with details.
 *   - An empty problem (B*S*H == 0) returns SAGE_OK without launching.
 *   - Inputs must be finite (and, with smooth_k, K - k_mean finite in float);
 *     other values give unspecified codes.
 *
 * Quantized layouts (written by sage_prepare, read by sage_attn). With
 * S_pad = sage_padded_len(S) (S rounded up to whole key tiles of
 * sage_kv_tile() = 128 keys) and NB = S_pad / 32:
 *   q8, k8      int8   [B][H][S_pad][128]  rows >= S are zero
 *   q_scale,    float  [B][H][NB]          scale of 32-row block n (codes *
 *   k_scale                                 scale ~ value); blocks >= ceil(S/32) are 0
 *   v8t         uint8  [B][H][128][S_pad]  OCP FP8 E4M3 codes, channel-major
 *                                          (keys contiguous); keys >= S are 0
 *   v_scale     float  [B][H][128]         per-channel scale
 *   k_mean      float  [B][H][128]         smooth_k: the subtracted mean; else 0
 * Every array is dense; pointers must be 16-byte aligned.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SAGE_BF16 = 1, SAGE_F16 = 2, SAGE_F32 = 3 } sage_dtype;

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARGUMENT = 1,
  SAGE_ERR_UNSUPPORTED = 2,
  SAGE_ERR_WORKSPACE_TOO_SMALL = 3,
  SAGE_ERR_DEVICE = 4
} sage_status;

/* A strided 4-D tensor on the device. Logical dimensions are (B, S, H, D);
 * strides are in elements, so [B,S,H,D] ("NHD") and [B,H,S,D] ("HND")
 * memory orders are both expressible. stride[3] must be 1. */
typedef struct {
  void* data;
  int32_t dtype; /* sage_dtype */
  int64_t size[4];
  int64_t stride[4];
} sage_tensor;

/* Keys per online-softmax tile (128). The pages fix an online softmax in
 * FP32 with P requantized to FP8 (issue, "The kernel") but not its tile size;
 * 128 is this library's convention, and it is part of the result: P is
 * requantized against the running maximum after each tile. */
int sage_kv_tile(void);

/* Library convention (layouts above): S rounded up to a multiple of
 * sage_kv_tile(); 0 for S <= 0, -1 when the rounded value does not fit in
 * int64. */
int64_t sage_padded_len(int64_t S);

/* Library convention (the caller owns every buffer): the device workspace
 * sage_prepare needs (per-chunk channel statistics); 0 for an empty or
 * unsupported problem (non-positive size, D not 64 or 128, or a problem past
 * the limits of validation step 2). */
size_t sage_prepare_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int smooth_k);

/* The prologue (issue, "The kernel"; release notes, "What changed"):
 *   k_mean[b,h,d] = float( fp64(sum_s K[b,s,h,d]) / S )   (smooth_k; else 0)
 *     where fp64(sum) is the exact sum rounded once to double (nearest, ties
 *     to even): "summed in fp64", independent of the order of the terms
 *   Q, K' = K - k_mean: per 32-row block a = max|x|, scale = a/127,
 *     code = rint(x * (127/a)) in [-127, 127] (ties to even; a = 0 gives 0)
 *   V: per channel a = max_s |V|, scale = a/448, code = E4M3(v * (448/a))
 *     (round to nearest even; an all-zero channel gives scale 0, codes 0)
 *   A block or channel with a < 2^-64, whose quotient 127/a or 448/a could
 *   exceed the largest float, is multiplied by 2^64 (exactly) together with a
 *   before the quotient is formed; wherever the quotient is finite this
 *   changes no code. The scale stays a/127 (a/448) of the unscaled a.
 * q, k, v: BF16 tensors of equal size with D = 128 (or 64). Outputs in the
 * layouts above; k_mean may be NULL. ws: device memory of at least
 * sage_prepare_workspace_bytes() bytes, contents need not be initialised.
 * Domain: finite inputs and, with smooth_k, K - k_mean finite in float (true
 * whenever |K| <= 2^126). On it the result is deterministic and every output
 * (codes, scales, k_mean) matches the CPU oracle bit for bit; outside it the
 * codes are unspecified. */
sage_status sage_prepare(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, int smooth_k, int8_t* q8,
                         float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t, float* v_scale, float* k_mean,
                         void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid allocation): sage_prepare
 * without the workspace argument. The prologue's statistics go to a static
 * device buffer of SAGE_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds
 * on each GPU it runs on until the process ends; the call allocates and frees
 * nothing. Same arguments (minus ws, ws_bytes), outputs, validation order and
 * results as sage_prepare; a problem whose sage_prepare_workspace_bytes()
 * exceeds the buffer returns SAGE_ERR_WORKSPACE_TOO_SMALL before any device
 * call. Every call on one GPU uses the same buffer, which keeps the last
 * call's contents (no call relies on them): calls that overlap on one GPU (two
 * streams, or unordered host threads) race and give undefined results. */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
sage_status sage_prepare_noalloc(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, int smooth_k,
                                 int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t, float* v_scale,
                                 float* k_mean, void* stream);

/* The attention step (issue, "The kernel") on sage_prepare's outputs:
 *   t_ij = float(q8_i . k8_j) * ((q_scale[i/32] * k_scale[j/32]) * (sm_scale * log2 e))
 *   online softmax in FP32 over key tiles of sage_kv_tile() keys in ascending
 *   order (running max m, alpha = 2^(m - m'), l from unrounded p),
 *   P requantized to E4M3 as E4M3(448 p) against the running max,
 *   PV in FP8 with FP32 accumulation,
 *   O[b,s,h,d] = BF16( o_d * v_scale[d] / (448 l) ).
 * o: BF16 tensor of logical size (B, S, H, 128), any 16-byte aligned strides
 * with stride[3] = 1. sm_scale > 0 and finite. */
sage_status sage_attn(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                      const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                      float sm_scale, const sage_tensor* o, void* stream);

/* sage_attn that also writes each row's log-sum-exp, an extension beyond the
 * pages (whose sageattn rejects return_lse): the natural log of the softmax
 * normaliser of the dequantized scores s_ij = t_ij ln 2, taken from the final
 * running maximum m and l as  lse[b][h][s] = m ln 2 + ln l  (fp32, [B][H][S]
 * contiguous, 4-byte aligned, caller-owned; NULL -> SAGE_ERR_INVALID_ARGUMENT).
 * With smooth_k the scores are those against the mean-subtracted keys, as the
 * softmax's are: they differ from the unsmoothed scores by sm_scale * q_i . k_mean
 * per row, which a caller merging partial results across key shards must add. */
sage_status sage_attn_lse(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                          const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                          float sm_scale, const sage_tensor* o, float* lse, void* stream);

/* sage_attn with both extensions selectable: is_causal != 0 masks key j for
 * query i when j > i (the usual causal mask for equal query and key lengths;
 * the key tiles still start at key 0, so row i is exactly the non-causal
 * computation over keys 0 .. i), and a non-NULL lse receives the rows'
 * log-sum-exp as in sage_attn_lse (over the keys the row sees). lse = NULL
 * writes none. Same layouts, alignment and errors as sage_attn. */
sage_status sage_attn_ex(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                         const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                         float sm_scale, int is_causal, const sage_tensor* o, float* lse, void* stream);

/* Library convention (the caller owns every buffer): the device workspace
 * sage_attn_fused needs, i.e. the quantized tensors, their scales and the
 * prologue's statistics; 0 when sage_prepare_workspace_bytes would be 0. */
size_t sage_fused_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D);

/* sage_prepare then sage_attn on one stream: the C image of
 * sageattn(q, k, v, tensor_layout, is_causal, sm_scale, return_lse) (issue,
 * "What I have so far"). is_causal != 0 selects the causal mask of sage_attn_ex
 * (an extension: the pages' package rejects it). return_lse = 1 also writes lse
 * as sage_attn_lse does (lse non-NULL); return_lse = 0 requires lse NULL (else
 * SAGE_ERR_INVALID_ARGUMENT). o and lse are bit for bit those of sage_prepare
 * followed by sage_attn_ex. Library convention: heads of at most 384 rows (768
 * at head dim 64) are handled in one launch that keeps the codes on chip; the
 * workspace's contents after a call are unspecified. */
sage_status sage_attn_fused(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, const sage_tensor* o,
                            int is_causal, float sm_scale, int return_lse, float* lse, int smooth_k, void* ws,
                            size_t ws_bytes, void* stream);

/* Library convention: the name of a status code. Errors are returned, never
 * handled another way, as the issue's package raises instead of falling back
 * ("What I have so far"). */
const char* sage_status_string(sage_status s);

/* Library convention: thread-local detail of the last error returned on this
 * thread ("" if none). */
const char* sage_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
