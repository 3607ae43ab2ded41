// Quantized attention forward on gfx950 (CDNA4): INT8 QK^T on MFMA, exp2
// online softmax in FP32, P requantized to OCP FP8 E4M3, FP8 PV on MFMA, BF16
// output. Method: kernels-community issue "aiter-sage-attention", section
// "The kernel" (QK^T in INT8 and PV in FP8 with FP32 accumulation; Q/K per
// 32-row block, V per channel).
//
// Work decomposition
//   workgroup = 4 waves = 128 queries of one (b, h); wave = 32 queries, i.e.
//   exactly one INT8 query block, so q_scale is uniform per wave.
//   Keys are consumed in tiles of 128 (the online-softmax tile, part of the
//   result's definition): per tile the wave computes 32x128 scores, one
//   running-max update, and 32x128 FP8 P times the 128x128 V tile.
//
// MFMA data flow (lane l, half h = l / 32, query column l % 32)
//   scores as S^T = K . Q^T with v_mfma_i32_32x32x32_i8: A = K rows, B = Q^T.
//   The accumulator of a 32x32 MFMA gives lane l rows 8(v/4) + 4h + v%4; the
//   A rows are fed in the permuted key order pi(r) = 16((r/4)%2) + 4(r/8) + r%4,
//   so lane l ends up holding keys 16h + v (v = 0..15) of every 32-key block
//   for its own query: contiguous keys, one query per lane.
//   PV as O^T = V^T . P^T with v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3): the
//   B operand (P^T) is exactly the lane's own packed probabilities (k-slot j of
//   half h is key 32(j/16) + 16h + j%16 of a 64-key half-tile), and the A
//   operand reads the matching keys of V's channel-major rows from LDS. No
//   cross-lane movement of P is needed.
//   The O^T accumulator gives lane l channels 32*blk + 8(v/4) + 4h + v%4 of its
//   query, so the per-query softmax state (m, l, alpha) is lane-local (the two
//   halves combine with one xor-32 exchange).
//
// LDS (32 KB per workgroup): K tile [128 keys][128 B], V tile [128 ch][128 B],
// filled by direct global->LDS DMA (16 B per lane). 16-byte chunks are XOR
// swizzled by (row & 7) (K: by the permuted row's low bits, which equal lane & 7)
// so the ds_read_b128 of 8 consecutive lanes hit 8 different bank groups.
#include "sage_internal.hpp"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPerWg = 32 * kWaves;
constexpr int kLdsK = 0;
constexpr int kLdsV = kKvTile * kHeadDim;   // 16 KB
constexpr int kLdsBytes = 2 * kKvTile * kHeadDim;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448): folds the P scale into exp2

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Global -> LDS copy of one K tile (128 keys x 128 B, contiguous in k8) and one
// V tile (128 channels x 128 keys, rows S_pad apart in v8t). Each wave moves
// 4 KB of each: instruction i of wave w fills LDS rows 8(4w+i) .. +8, lane t
// landing at byte 16 t of that 1 KB; the lane fetches the global chunk that
// belongs at its swizzled position.
__device__ inline void load_tile(uint8_t* lds, const int8_t* kg, const uint8_t* vg, int64_t S_pad, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    const int pc = lane & 7;
    const int kc = pc ^ (row & 7);   // K rows are stored in natural key order, swizzled by key & 7
    __builtin_amdgcn_global_load_lds(kg + row * kHeadDim + kc * 16, LDS_PTR(lds + kLdsK + 1024 * (4 * wave + i)), 16,
                                     0, 0);
    const int vc = pc ^ (row & 7);
    __builtin_amdgcn_global_load_lds(vg + (int64_t)row * S_pad + vc * 16,
                                     LDS_PTR(lds + kLdsV + 1024 * (4 * wave + i)), 16, 0, 0);
  }
}

__device__ inline uint32_t pack_bf16x2(float a, float b) { return f32_to_bf16(a) | (f32_to_bf16(b) << 16); }

__global__ void __launch_bounds__(kThreads, 2)
attn_kernel(const int8_t* __restrict__ q8, const float* __restrict__ q_scale, const int8_t* __restrict__ k8,
            const float* __restrict__ k_scale, const uint8_t* __restrict__ v8t, const float* __restrict__ v_scale,
            int64_t H, int64_t S, int64_t S_pad, int64_t nqt, int64_t nwg, float sl2, Bf16OutView o) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
  // give each XCD a contiguous range of (head, query tile) so the query tiles
  // of one head share that XCD's L2 while they stream the same K/V.
  const int64_t bid = blockIdx.x;
  const int64_t per = nwg / 8, rem = nwg % 8, x = bid % 8;
  const int64_t logical = x * per + (x < rem ? x : rem) + bid / 8;
  const int64_t bh = logical / nqt, qt = logical % nqt;
  const int64_t b = bh / H, h = bh % H;

  const int64_t q0 = qt * kQPerWg + 32 * wave;   // this wave's first query (one INT8 block)
  const int8_t* kg = k8 + bh * S_pad * kHeadDim;
  const uint8_t* vg = v8t + bh * kHeadDim * S_pad;
  const float* ks = k_scale + bh * (S_pad / kQBlock);
  const float qs = q_scale[bh * (S_pad / kQBlock) + q0 / kQBlock];

  // B operand of the score MFMAs: Q^T column = this lane's query, k-slots
  // 16h..16h+15 of each 32-channel step.
  v4i qreg[4];
  {
    const int8_t* qrow = q8 + (bh * S_pad + q0 + col) * kHeadDim + 16 * half;
#pragma unroll
    for (int s = 0; s < 4; ++s) qreg[s] = *reinterpret_cast<const v4i*>(qrow + 32 * s);
  }

  // A-operand row of the score MFMA fed by this lane: key pi(col) of a 32-key block
  const int prow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  v16f oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  const int64_t ntiles = S_pad / kKvTile;
  for (int64_t t = 0; t < ntiles; ++t) {
    const int64_t key0 = t * kKvTile;
    __syncthreads();   // previous tile's LDS reads are done
    load_tile(lds, kg + key0 * kHeadDim, vg + key0, S_pad, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- scores: 4 blocks of 32 keys x 32 queries
    v16i sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      v16i acc = {};
      const int krow = 32 * kb + prow;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int chunk = (2 * s + half) ^ (krow & 7);
        v4i a = *reinterpret_cast<const v4i*>(lds + kLdsK + krow * kHeadDim + chunk * 16);
        acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[s], acc, 0, 0, 0);
      }
      sacc[kb] = acc;
    }

    // ---- online softmax (exp2 domain, per-block dequant constant)
    float cblk[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cblk[kb] = (qs * ks[key0 / kQBlock + kb]) * sl2;
    const bool tail = key0 + kKvTile > S;
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      int im = INT32_MIN;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t key = key0 + 32 * kb + 16 * half + v;
        int a = sacc[kb][v];
        if (tail && key >= S) a = INT32_MIN;
        im = max(im, a);
      }
      // max over a block = (float)(max code dot) * c since c >= 0 and rounding is monotone
      if (im != INT32_MIN) tmax = fmaxf(tmax, (float)im * cblk[kb]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
    const float moff = m_new - kLog2_448;                        // exp2(t - moff) = 448 p

    float psum = 0.0f;
    v8i pk[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; v += 4) {
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sacc[kb][v + u], cblk[kb], -moff));
          if (tail && key0 + 32 * kb + 16 * half + v + u >= S) p[u] = 0.0f;
          psum += p[u];
        }
        const int j = 16 * (kb & 1) + v;   // k-slot of p[0] within the 64-key half-tile
        int dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], dw, true);
        pk[kb >> 1][j >> 2] = dw;
      }
    }
    l_run = alpha * l_run + psum;   // l carries the factor 448
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha;
    }
    m_run = m_new;

    // ---- PV: O^T[ch][q] += V^T[ch][key] P^T[key][q], two 64-key halves
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int ch = 32 * d + col;
        const uint8_t* vrow = lds + kLdsV + ch * kKvTile;
        const int c1 = (4 * kc + half) ^ (ch & 7), c2 = (4 * kc + 2 + half) ^ (ch & 7);
        v4i a0 = *reinterpret_cast<const v4i*>(vrow + c1 * 16);
        v4i a1 = *reinterpret_cast<const v4i*>(vrow + c2 * 16);
        v8i a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pk[kc], oacc[d], 0, 0, 0, 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = o * v_scale / (448 l)
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.0f / l_tot;
  const int64_t qi = q0 + col;
  if (qi < S) {
    uint16_t* orow = o.data + b * o.sb + qi * o.ss + h * o.sh;
    const float* vs = v_scale + bh * kHeadDim;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ch = 32 * d + 8 * a + 4 * half;
        const float4 sc = *reinterpret_cast<const float4*>(vs + ch);
        uint2 w;
        w.x = pack_bf16x2(oacc[d][4 * a + 0] * sc.x * inv_l, oacc[d][4 * a + 1] * sc.y * inv_l);
        w.y = pack_bf16x2(oacc[d][4 * a + 2] * sc.z * inv_l, oacc[d][4 * a + 3] * sc.w * inv_l);
        *reinterpret_cast<uint2*>(orow + ch) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_attention(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                            const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H,
                            float sm_scale, const Bf16OutView& o, hipStream_t stream) {
  const int64_t S_pad = padded_len(S);
  const int64_t nqt = S_pad / kQPerWg;
  const int64_t nwg = B * H * nqt;
  const float sl2 = sm_scale * kLog2e;
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream, q8, q_scale, k8, k_scale, v8t,
                     v_scale, H, S, S_pad, nqt, nwg, sl2, o);
  return hipGetLastError();
}

}  // namespace sage
