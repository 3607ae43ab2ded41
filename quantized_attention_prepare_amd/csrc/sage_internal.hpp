// Internal declarations shared by the library's HIP sources (not installed).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int kHeadDim = 128;   // the head dim of the pages' workloads; 64 is the other one built
inline bool supported_head_dim(int64_t D) { return D == 64 || D == 128; }
constexpr int kKvTile = 128;    // keys per online-softmax tile
constexpr int kQBlock = 32;     // rows per INT8 quantization block
constexpr int kChunk = 128;     // rows handled by one prologue workgroup pass
// Longest sequence: a head's quantized K or V (S_pad * 128 bytes) must stay
// below 4 GiB, the 32-bit byte extent of the attention kernel's buffer
// resources; 2^25 - 128 rows is the largest whole number of key tiles under it.
constexpr int64_t kMaxSeq = (int64_t(1) << 25) - kKvTile;
// B * H * S_pad / 128 bounds every launch's workgroup count (one per 128-row
// chunk or query tile of a head); it must fit a 32-bit signed grid size.
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;

// S rounded up to whole key tiles; 0 for S <= 0, -1 when that does not fit int64.
inline int64_t padded_len(int64_t S) {
  if (S <= 0) return 0;
  const int64_t tiles = S / kKvTile + (S % kKvTile != 0);
  return tiles > INT64_MAX / kKvTile ? -1 : tiles * kKvTile;
}

// Strided BF16 input view: element (b, s, h, d) at data[b*sb + s*ss + h*sh + d].
struct Bf16View {
  const uint16_t* data;
  int64_t sb, ss, sh;
};

struct Bf16OutView {
  uint16_t* data;
  int64_t sb, ss, sh;
};

// Workspace layout of the prologue (per-chunk statistics and per-head results).
struct PrologueWs {
  double* ksum_part;   // [B*H][nparts][128]
  float* vmax_part;    // [B*H][nparts][128]
  float* kmean;        // [B*H][128]
  float* vinv;         // [B*H][128]  448 / (amax * lift)
  float* vlift;        // [B*H][128]  2^64 for a channel with amax < 2^-64, else 1
};

struct PrologueShape {
  int64_t B, S, H, D, S_pad;
  int chunks_per_wg;   // 128-row chunks folded into one statistics workgroup
  int64_t nparts;      // statistics partials per head
};

PrologueShape prologue_shape(int64_t B, int64_t S, int64_t H, int64_t D);
size_t prologue_ws_bytes(const PrologueShape& ps);
PrologueWs prologue_ws_carve(void* ws, const PrologueShape& ps);

hipError_t launch_prologue(const Bf16View& q, const Bf16View& k, const Bf16View& v, const PrologueShape& ps,
                           int smooth_k, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t,
                           float* v_scale, float* k_mean_out, const PrologueWs& ws, hipStream_t stream);

hipError_t launch_attention(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                            const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                            float sm_scale, bool causal, const Bf16OutView& o, float* lse, hipStream_t stream);

// The whole forward in one launch for short heads (one workgroup per head; the
// codes and scales never leave LDS): whether a head of S rows fits, and the
// launch.
bool short_fused_fits(int64_t S, int64_t D);
hipError_t launch_fused_short(const Bf16View& q, const Bf16View& k, const Bf16View& v, int64_t B, int64_t S,
                              int64_t H, int64_t D, int smooth_k, float sm_scale, bool causal, const Bf16OutView& o,
                              float* lse, hipStream_t stream);

// ---------------------------------------------------------------- device helpers
__device__ inline float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// float -> BF16 bits, round to nearest even (inputs are finite).
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace sage
