// Device helpers of the prologue's passes, shared by the prologue kernels and
// the one-workgroup-per-head form of the whole forward for short heads: 16-byte
// BF16 row loads, the INT8 block quantization, the checked fp64 addition and
// the exact channel sums.
//
// Method: kernels-community issue "aiter-sage-attention" (section "The
// kernel": Q/K per 32-row block, V per channel) and the SageAttention-RDNA4
// v0.4.0 release notes ("What changed": key mean summed in fp64).
#pragma once
#include "sage_internal.hpp"

namespace sage {
namespace {

struct Row16 { uint32_t w[4]; };            // 16 bytes = 8 BF16 channels

__device__ inline Row16 load16(const uint16_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return Row16{{u.x, u.y, u.z, u.w}};
}
// Streaming hints. Q is read once, so its loads are nontemporal: it need not
// take room in the caches that the quantize pass's second read of K and V
// hits (2-3 % faster on long sequences; the same hint on K or V loses). The
// INT8 and E4M3 codes are written with nontemporal stores: the prologue never
// reads them back, and streaming stores leave the caches to its reads (10 %
// faster on a 28-head 32k-token call, 5 % at 40 heads x 75k tokens, no change
// on short calls). Hints change no value.
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
__device__ inline Row16 load16nt(const uint16_t* p) {
  v4u_t u = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
  return Row16{{u[0], u[1], u[2], u[3]}};
}

__device__ inline void unpack(const Row16& r, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(r.w[i]); x[2 * i + 1] = bf16_hi(r.w[i]); }
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

constexpr float kTiny = 0x1p-64f;       // blocks and channels below this absmax are lifted
constexpr float kTinyLift = 0x1p64f;    // by this exact factor before 127/a or 448/a

// a + b when that sum is a double, else NaN (which every later addition keeps).
// If the sum is exact, s - a = b and s - b = a exactly. If it is not, then for
// the operand of larger magnitude, say a, s - a is computed exactly (it
// recovers the rounding error of s, Dekker's Fast2Sum) and differs from b.
// Summing key channels with it in any order therefore gives either the exact
// sum, which is then also the sum rounded once, or NaN.
__device__ inline double add_exact_or_nan(double a, double b) {
  const double s = a + b;
  return (s - a == b && s - b == a) ? s : __longlong_as_double(0x7FF8000000000000ll);
}

// Lane geometry of one wave over a 32-row block of D channels: lane (c, g),
// c = lane % L, g = lane / L, holds channels 8c .. 8c+7 of rows G*i + g,
// i = 0 .. I-1 (L lanes per row, G row groups, I rows per lane).
template <int D>
struct Geo {
  static constexpr int L = D / 8;
  static constexpr int G = 64 / L;
  static constexpr int I = 32 / G;
};

// Quantize one 32-row x D-channel block held as x[i*8+e] = element
// (row G*i + g, channel 8c + e); invalid rows hold 0.
// Writes the 32 rows of codes and the block's scale.
template <int D>
__device__ inline void quant_block_store(float (&x)[8 * Geo<D>::I], int8_t* dst_rows, float* scale_out,
                                         int lane) {
  using Gm = Geo<D>;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8 * Gm::I; ++i) a = fmaxf(a, fabsf(x[i]));
  a = wave_max(a);
  float scale = 0.0f, inv = 0.0f;
  if (a != 0.0f) {
    scale = a / 127.0f;   // correctly rounded IEEE division
    // A block of tiny values (a < 2^-64, where 127/a may exceed the largest
    // float) is lifted by 2^64, exactly, before the quotient is formed; the
    // codes are those of the unlifted form wherever its quotient is finite.
    // The branch is uniform over the wave (a is the block's maximum).
    if (a < kTiny) {
#pragma unroll
      for (int i = 0; i < 8 * Gm::I; ++i) x[i] *= kTinyLift;
      inv = 127.0f / (a * kTinyLift);
    } else {
      inv = 127.0f / a;
    }
  }
  const int c = lane % Gm::L, g = lane / Gm::L;
#pragma unroll
  for (int i = 0; i < Gm::I; ++i) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(x[i * 8 + e] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      uint32_t byte = (uint32_t)(int32_t)r & 0xFFu;
      if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
    }
    __builtin_nontemporal_store(v2u_t{lo, hi}, reinterpret_cast<v2u_t*>(dst_rows + (int64_t)(Gm::G * i + g) * D + 8 * c));
  }
  if (lane == 0) *scale_out = scale;
}

// The same quantization as quant_block_store, step for step, with the codes
// returned instead of stored (for a caller that places them in LDS): row
// G*i + g's codes of channels 8c..8c+3 in lo[i], 8c+4..8c+7 in hi[i]; returns
// the scale.
template <int D>
__device__ inline float quant_block_codes(float (&x)[8 * Geo<D>::I], uint32_t (&lo)[Geo<D>::I],
                                          uint32_t (&hi)[Geo<D>::I]) {
  using Gm = Geo<D>;
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8 * Gm::I; ++i) a = fmaxf(a, fabsf(x[i]));
  a = wave_max(a);
  float scale = 0.0f, inv = 0.0f;
  if (a != 0.0f) {
    scale = a / 127.0f;
    if (a < kTiny) {   // lifted as in quant_block_store
#pragma unroll
      for (int i = 0; i < 8 * Gm::I; ++i) x[i] *= kTinyLift;
      inv = 127.0f / (a * kTinyLift);
    } else {
      inv = 127.0f / a;
    }
  }
#pragma unroll
  for (int i = 0; i < Gm::I; ++i) {
    uint32_t l = 0, h = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(x[i * 8 + e] * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      uint32_t byte = (uint32_t)(int32_t)r & 0xFFu;
      if (e < 4) l |= byte << (8 * e); else h |= byte << (8 * (e - 4));
    }
    lo[i] = l;
    hi[i] = h;
  }
  return scale;
}

// Exact channel sums: a finite BF16 value is M * 2^(e - 133) with integers
// 0 <= M < 256 and 0 <= e <= 253 (exponent field E > 0: M = 128 + mantissa,
// e = E - 1; E = 0: M = mantissa, e = 0), so a channel's sum over fewer than
// 2^25 rows is an integer multiple of 2^-133 below 2^286 in magnitude: nine
// 32-bit digits of a two's complement integer hold it.
constexpr int kDigits = 9;

// Threads of this many slices form the exact sums (their digit words share
// the workgroup's LDS with the fold of the partials).
constexpr int kExactSlices = 4;

// Channel d's exact key sum over rows s = j, j + kExactSlices, ..., accumulated
// by thread (d, j) into its own 64-bit words w(j, 0..8, d) (one word per 32-bit
// digit, carries left for later: a word receives at most 2^23 additions below
// 2^32 each); the caller adds the slices and rounds.
__device__ inline void exact_sum_rows(const uint16_t* kcol, int64_t ss, int64_t S, int j, long long* dig_j_d,
                                      int dstride) {
  for (int64_t s = j; s < S; s += kExactSlices) {
    const uint32_t b = kcol[s * ss];
    const uint32_t E = (b >> 7) & 0xFFu, M = E ? 128u + (b & 0x7Fu) : (b & 0x7Fu);
    if (M == 0) continue;
    const int e = E ? (int)E - 1 : 0;
    const unsigned long long w = (unsigned long long)M << (e & 31);   // below 2^39
    long long lo = (long long)(w & 0xFFFFFFFFull), hi = (long long)(w >> 32);
    if (b & 0x8000u) { lo = -lo; hi = -hi; }
    dig_j_d[(e >> 5) * dstride] += lo;
    dig_j_d[((e >> 5) + 1) * dstride] += hi;
  }
}

// The integer sum_k w[k] 2^(32k) (w[k] the digit words of all slices added,
// each below 2^57 in magnitude) times 2^-133, rounded once to double.
// Fully unrolled, so the digits stay in registers.
__device__ inline double digits_to_double(const long long (&w)[kDigits]) {
  uint32_t dig[kDigits];
  long long carry = 0;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    const long long t = w[k] + carry;
    dig[k] = (uint32_t)(t & 0xFFFFFFFFll);
    carry = t >> 32;   // arithmetic shift: floor division by 2^32
  }
  // carry is now the sign extension above 288 bits: 0 or -1
  const bool negative = carry < 0;
  if (negative) {   // two's complement negation of the 288-bit integer
    unsigned long long c = 1;
#pragma unroll
    for (int k = 0; k < kDigits; ++k) {
      const unsigned long long t = (unsigned long long)(~dig[k]) + c;
      dig[k] = (uint32_t)t;
      c = t >> 32;
    }
  }
  int top = -1;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) top = dig[k] != 0 ? k : top;
  if (top < 0) return 0.0;
  // The 64 bits from the most significant one down, from digits top, top - 1
  // and top - 2, with every bit below them ORed into bit 0 (below the rounding
  // position of a 53-bit significand, so the conversion rounds once, correctly).
  unsigned long long hi = 0, mid = 0, lo = 0;
  bool sticky = false;
#pragma unroll
  for (int k = 0; k < kDigits; ++k) {
    hi = k == top ? dig[k] : hi;
    mid = k == top - 1 ? dig[k] : mid;
    lo = k == top - 2 ? dig[k] : lo;
    sticky |= k < top - 2 && dig[k] != 0;
  }
  const int msb = 31 - __clz((int)hi);
  unsigned long long u = (hi << (63 - msb)) | (mid << (31 - msb)) | (lo >> (msb + 1));
  sticky |= (lo & ((1ull << (msb + 1)) - 1)) != 0;
  u |= sticky ? 1ull : 0ull;
  const int low_bit = 32 * (top - 2) + msb + 1;   // weight of u's bit 0, in units of 2^-133
  const double m = ldexp((double)u, low_bit - 133);
  return negative ? -m : m;
}

}  // namespace
}  // namespace sage
