// Quantized attention forward on gfx950 (CDNA4): INT8 QK^T on MFMA, exp2
// online softmax in FP32, P requantized to OCP FP8 E4M3, FP8 PV on MFMA, BF16
// output. Method: kernels-community issue "aiter-sage-attention", section
// "The kernel" (QK^T in INT8 and PV in FP8 with FP32 accumulation; Q/K per
// 32-row block, V per channel).
//
// Work decomposition
//   workgroup = 4 waves = 128 queries of one (b, h), two workgroups per CU;
//   wave = 32 queries, i.e. exactly one INT8 query block, so q_scale is
//   uniform per wave. Keys are consumed in tiles of 128 (the online-softmax
//   tile, part of the result's definition).
//
// Schedule (per wave, iteration t)
//   max of tile t's scores -> issue the INT8 score MFMAs of tile t+1 (their
//   results are not needed until the next iteration) -> exp2 / FP8 packing of
//   tile t while those MFMAs execute -> rescale O -> issue the FP8 PV MFMAs of
//   tile t, which run on into the next iteration's copy wait and max. The
//   matrix cores thus work under the same wave's softmax; the other workgroup
//   on the CU, unsynchronised with this one, fills the remaining gaps.
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
// LDS (80 KB per workgroup): two K tiles [128 keys][128 B] and two V tiles
// [128 ch][128 B] (tile t in buffer t & 1), filled by buffer loads that write
// LDS directly, and the workgroup's 128 INT8 query rows. During iteration t
// the wave reads K(t+1) and V(t) while K(t+2) and V(t+1) are being copied.
// Bank layout: gfx950 serves a ds_read_b128 16 lanes at a time from 64 banks of
// 4 bytes, so 16 consecutive lanes must hit 16 different 16-byte slots of a
// 256-byte bank row. Rows are 128 bytes (two rows per bank row) and the 16-byte
// chunk c of row r is stored at c XOR f(r): for V and Q rows f(r) = (r>>1)&7;
// for K, whose rows are read in the permuted order pi,
// f(r) = ((r>>1)&3) | ((r>>4)&1)<<2.
#include "sage_internal.hpp"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kCopyInstr = 16 / kWaves;   // 1 KB copy instructions per wave per 16 KB tile
constexpr int kThreads = 64 * kWaves;
constexpr int kQPerWg = 32 * kWaves;
constexpr int kTileBytes = kKvTile * kHeadDim;   // 16 KB: one K or V tile
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448): folds the P scale into exp2
constexpr int kBufferWord3 = 0x00020000;          // raw (untyped) buffer access

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define SAGE_INLINE __device__ __attribute__((always_inline)) inline

// Global -> LDS copies with buffer loads that write LDS directly (16 B per
// lane). Each wave moves 4 KB of a 16 KB tile: instruction i of wave w fills
// LDS rows r = 8(4w+i) + lane/8, lane t landing at byte 16 t of that 1 KB. The
// lane fetches the global chunk that belongs at its swizzled position, chunk
// (lane % 8) XOR f(r); f(r) depends only on the lane and on (w, i), so each
// instruction's lane offset is a per-lane constant. One buffer resource per head
// holds the 64-bit base and the exact byte extent (the hardware bounds-checks
// every copy); tile and row offsets go in the 32-bit scalar offset and the
// lane offset in one vector register.
// K tile t: 128 keys x 128 B, contiguous in k8 (head extent S_pad * 128 B).
SAGE_INLINE void load_k(uint8_t* dst, __amdgpu_buffer_rsrc_t rk, int t, const uint32_t (&lane_off)[kCopyInstr],
                        int wave) {
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS_PTR(dst + 1024 * (kCopyInstr * wave + i)), 16, lane_off[i],
                                             (uint32_t)t * kTileBytes + 1024u * (kCopyInstr * wave + i), 0, 0);
}
// V tile t: 128 channels x 128 keys; channel rows are S_pad bytes apart in v8t
// (head extent 128 * S_pad B).
SAGE_INLINE void load_v(uint8_t* dst, __amdgpu_buffer_rsrc_t rv, int t, uint32_t S_pad,
                        const uint32_t (&lane_off)[kCopyInstr], int wave) {
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, LDS_PTR(dst + 1024 * (kCopyInstr * wave + i)), 16, lane_off[i],
                                             (uint32_t)t * kKvTile + (uint32_t)(8 * (kCopyInstr * wave + i)) * S_pad,
                                             0, 0);
}

SAGE_INLINE uint32_t pack_bf16x2(float a, float b) { return f32_to_bf16(a) | (f32_to_bf16(b) << 16); }

// max over the two lanes l and l ^ 32 (the two halves of one query's keys):
// v_permlane32_swap with the same value in both operands returns the upper
// halves swapped with the lower ones, so the pair holds both values on every
// lane.
SAGE_INLINE float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Per-wave online-softmax state and output accumulators.
struct WaveState {
  v16f oacc[4];   // O^T blocks: channels 32*d + 8(v/4) + 4h + v%4 of this lane's query
  v16i sacc[4];   // scores of the tile whose softmax is next (4 blocks of 32 keys)
  v8i pk[2];      // FP8 probabilities of the tile whose PV is next (two 64-key halves)
  float m_run;    // running max (log2 units)
  float l_run;    // this lane-half's share of 448 * sum p
};

// PV of one tile: O^T[ch][q] += V^T[ch][key] P^T[key][q] over two 64-key
// halves; the four output channel blocks are independent MFMAs.
SAGE_INLINE void pv_tile(WaveState& st, const uint8_t* vbuf, int half, int col) {
  const int fv = (col >> 1) & 7;   // f(ch) for ch = 32 d + col: 32 d does not change bits 1-3
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint8_t* vrow = vbuf + (32 * d + col) * kKvTile;
      union { v8i v; v4i q[2]; } a;
      a.q[0] = *reinterpret_cast<const v4i*>(vrow + (((4 * kc + half) ^ fv) * 16));
      a.q[1] = *reinterpret_cast<const v4i*>(vrow + (((4 * kc + 2 + half) ^ fv) * 16));
      st.oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.v, st.pk[kc], st.oacc[d], 0, 0, 0, 0, 0, 0);
    }
  }
}

// INT8 scores S^T = K . Q^T of one tile into sacc: row pi(col) of each 32-key
// block, channels 32s + 16h .. +15; the four score blocks are independent
// MFMAs.
SAGE_INLINE void qk_tile(v16i (&sacc)[4], const uint8_t* kbuf, const uint8_t* qrow, int half, int col, int prow) {
  const uint8_t* krow = kbuf + prow * kHeadDim;
  const int fk = ((prow >> 1) & 3) | (((prow >> 4) & 1) << 2);   // f(32 kb + prow) for every kb
  const int fq = (col >> 1) & 7;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const v4i qb = *reinterpret_cast<const v4i*>(qrow + (((2 * s + half) ^ fq) * 16));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const v4i a = *reinterpret_cast<const v4i*>(krow + 32 * kb * kHeadDim + (((2 * s + half) ^ fk) * 16));
      if (s == 0) {
        const v16i z = {};
        sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qb, z, 0, 0, 0);
      } else {
        sacc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qb, sacc[kb], 0, 0, 0);
      }
    }
  }
}

// Softmax step for one tile: issues the next tile's score MFMAs, then the
// online update of the running max and sum, FP8 probabilities into pk,
// rescale of O; on return sacc holds the next tile's scores.
// cblk[kb] = (q_scale * k_scale) * sm_scale * log2 e of the tile's 32-key
// blocks. nvalid < 128 marks a ragged last tile: the padded keys' scores are
// replaced with INT32_MIN (never above a valid score since |acc| <= 2^21),
// blocks made only of padding come with cblk = +inf (probability exactly 0),
// and in the partly padded block the padded keys' probability, which only
// matters for l (their V codes are 0), is subtracted from l afterwards.
SAGE_INLINE void softmax_step(WaveState& st, const float (&cblk)[4], int nvalid, int half, const uint8_t* kbuf_next,
                              const uint8_t* qrow, int col, int prow) {
  // the next tile's score MFMAs go out first and execute under this softmax
  v16i snext[4];
  qk_tile(snext, kbuf_next, qrow, half, col, prow);
  __builtin_amdgcn_sched_barrier(0);
  const int kbase = 16 * half;   // key offset of this lane's first key in each 32-key block
  if (nvalid < kKvTile) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * kb + kbase + v >= nvalid) st.sacc[kb][v] = INT32_MIN;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    int m8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) m8[v] = max(st.sacc[kb][v], st.sacc[kb][v + 8]);
    const int im = max(max(max(m8[0], m8[1]), max(m8[2], m8[3])), max(max(m8[4], m8[5]), max(m8[6], m8[7])));
    // the block max of t = float(acc) * c is float(max acc) * c because c >= 0
    // and rounding is monotone
    tmax = fmaxf(tmax, (float)im * cblk[kb]);
  }
  tmax = max_xor32(tmax);
  const float m_new = fmaxf(st.m_run, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 0 on the first tile
  const float moff = m_new - kLog2_448;                           // exp2(t - moff) = 448 p

  // 16 independent partial sums keep the additions off one serial chain
  float ps[4][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int v = 0; v < 16; v += 4) {
      float p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)st.sacc[kb][v + u], cblk[kb], -moff));
        ps[kb][u] = v == 0 ? p[u] : ps[kb][u] + p[u];
      }
      const int j = 16 * (kb & 1) + v;   // k-slot of p[0] within the 64-key half-tile
      int dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], dw, true);
      st.pk[kb >> 1][j >> 2] = dw;
    }
  }
  float psum = ((ps[0][0] + ps[0][1]) + (ps[0][2] + ps[0][3])) + ((ps[1][0] + ps[1][1]) + (ps[1][2] + ps[1][3])) +
               (((ps[2][0] + ps[2][1]) + (ps[2][2] + ps[2][3])) + ((ps[3][0] + ps[3][1]) + (ps[3][2] + ps[3][3])));
  if (nvalid < kKvTile && (nvalid & 31)) {
    const int kbp = nvalid >> 5;   // the partly padded block
    const int nmask = min(16, max(0, 32 * kbp + kbase + 16 - nvalid));
    const float pm = __builtin_amdgcn_exp2f(__builtin_fmaf((float)INT32_MIN, cblk[kbp], -moff));
    if (nmask > 0) psum -= (float)nmask * pm;
  }
  st.l_run = alpha * st.l_run + psum;
  // Unconditional: skipping it when every alpha is 1 would need a branch
  // around the accumulators, which costs more registers than the multiplies.
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) st.oacc[d][v] *= alpha;
  st.m_run = m_new;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) st.sacc[kb] = snext[kb];
}

__global__ void __launch_bounds__(kThreads, 2)
attn_kernel(const int8_t* __restrict__ q8, const float* __restrict__ q_scale, const int8_t* __restrict__ k8,
            const float* __restrict__ k_scale, const uint8_t* __restrict__ v8t, const float* __restrict__ v_scale,
            int64_t H, int64_t S, int64_t S_pad, int64_t nqt, int64_t nwg, float sl2, Bf16OutView o) {
  // two K and two V tile buffers (indexed by tile & 1), then the workgroup's
  // 128 query rows [query][128 B] (16-byte chunks XOR swizzled by query & 7)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kTileBytes + kQPerWg * kHeadDim];
#define KBUF(i) (lds + (i) * kTileBytes)
#define VBUF(i) (lds + (2 + (i)) * kTileBytes)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  // copy chunk of this lane: (lane % 8) XOR f(row) for row = 8 j + lane / 8, j = 4 wave + i
  uint32_t k_lane_off[kCopyInstr];
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i) {
    const int j = kCopyInstr * wave + i;
    k_lane_off[i] =
        (uint32_t)((lane >> 3) * kHeadDim + (((lane & 7) ^ (((lane >> 4) & 3) | (((j >> 1) & 1) << 2))) * 16));
  }

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
  // give each XCD a contiguous range of (head, query tile) so the query tiles
  // of one head share that XCD's L2 while they stream the same K/V.
  const int64_t bid = blockIdx.x;
  const int64_t per = nwg / 8, rem = nwg % 8, x = bid % 8;
  const int64_t logical = x * per + (x < rem ? x : rem) + bid / 8;
  const int64_t bh = logical / nqt, qt = logical % nqt;
  const int64_t b = bh / H, h = bh % H;

  const int64_t q0 = qt * kQPerWg + 32 * wave;   // this wave's first query (one INT8 block)
  const bool active = q0 < S_pad;                // the last workgroup may reach past S_pad
  const uint32_t spad32 = (uint32_t)S_pad;       // 128 S_pad < 2^32 (host check)
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k8 + bh * S_pad * kHeadDim), 0, (int)(spad32 * kHeadDim), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v8t + bh * kHeadDim * S_pad), 0, (int)(spad32 * kHeadDim), kBufferWord3);
  uint32_t v_lane_off[kCopyInstr];
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i)
    v_lane_off[i] = (uint32_t)(lane >> 3) * spad32 + (uint32_t)(((lane & 7) ^ (((lane >> 4) & 3) | ((i & 1) << 2))) * 16);
  const float* ks = k_scale + bh * (S_pad / kQBlock);
  const float qs = active ? q_scale[bh * (S_pad / kQBlock) + q0 / kQBlock] : 0.0f;

  // This wave's 32 query rows go to LDS once (zeros past S_pad); the score
  // MFMAs read their B operand from there.
  uint8_t* qlds = lds + 4 * kTileBytes + 32 * wave * kHeadDim;
  {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3), c = lane & 7;   // row r of the wave, 16-byte chunk c
      uint4 val = make_uint4(0, 0, 0, 0);
      if (active) val = *reinterpret_cast<const uint4*>(q8 + (bh * S_pad + q0 + r) * kHeadDim + c * 16);
      *reinterpret_cast<uint4*>(qlds + r * kHeadDim + ((c ^ ((r >> 1) & 7)) * 16)) = val;
    }
  }
  const uint8_t* qrow = qlds + col * kHeadDim;
  // A-operand row of the score MFMA fed by this lane: key pi(col) of a 32-key block
  const int prow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  WaveState st;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) st.oacc[d][v] = 0.0f;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) st.pk[kc][i] = 0;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;

  const int ntiles = (int)(S_pad / kKvTile);
  const int last_valid = (int)(S - (int64_t)(ntiles - 1) * kKvTile);   // valid keys in the last tile (1..128)

  // K(0), K(1), V(0) in; scores of tile 0.
  load_k(KBUF(0), rk, 0, k_lane_off, wave);
  if (ntiles > 1) load_k(KBUF(1), rk, 1, k_lane_off, wave);
  load_v(VBUF(0), rv, 0, spad32, v_lane_off, wave);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  qk_tile(st.sacc, KBUF(0), qrow, half, col, prow);
  float4 ksv = *reinterpret_cast<const float4*>(ks);   // k_scale of the four blocks of the current tile

  // Iteration t: softmax of tile t (with the scores of tile t+1 computed under
  // it), PV of tile t. On entry K(t+1) and V(t) must be in LDS; K(t+2) and
  // V(t+1) are copied into the buffers K(t) and V(t-1) occupied. After the last
  // tile the score MFMAs read stale K bytes whose scores are never used.
  for (int t = 0; t < ntiles; ++t) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed
    __syncthreads();                 // ... everyone's; K(t) and V(t-1) are no longer read
    if (t + 2 < ntiles) load_k(KBUF(t & 1), rk, t + 2, k_lane_off, wave);
    if (t + 1 < ntiles) load_v(VBUF((t + 1) & 1), rv, t + 1, spad32, v_lane_off, wave);
    const int nvalid = t == ntiles - 1 ? last_valid : kKvTile;
    const float kss[4] = {ksv.x, ksv.y, ksv.z, ksv.w};
    float cblk[4];   // (q_scale * k_scale) * sm_scale * log2 e; +inf for a block made only of padding
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) cblk[kb] = 32 * kb >= nvalid ? INFINITY : (qs * kss[kb]) * sl2;
    if (t + 1 < ntiles) ksv = *reinterpret_cast<const float4*>(ks + 4 * (t + 1));
    softmax_step(st, cblk, nvalid, half, KBUF((t + 1) & 1), qrow, col, prow);
    pv_tile(st, VBUF(t & 1), half, col);
  }

  // ---- epilogue: O = o * v_scale / (448 l)
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
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
        w.x = pack_bf16x2(st.oacc[d][4 * a + 0] * sc.x * inv_l, st.oacc[d][4 * a + 1] * sc.y * inv_l);
        w.y = pack_bf16x2(st.oacc[d][4 * a + 2] * sc.z * inv_l, st.oacc[d][4 * a + 3] * sc.w * inv_l);
        *reinterpret_cast<uint2*>(orow + ch) = w;
      }
    }
  }
#undef KBUF
#undef VBUF
}

}  // namespace

hipError_t launch_attention(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                            const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H,
                            float sm_scale, const Bf16OutView& o, hipStream_t stream) {
  const int64_t S_pad = padded_len(S);
  const int64_t nqt = (S_pad + kQPerWg - 1) / kQPerWg;
  const int64_t nwg = B * H * nqt;
  const float sl2 = sm_scale * kLog2e;
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream, q8, q_scale, k8, k_scale, v8t,
                     v_scale, H, S, S_pad, nqt, nwg, sl2, o);
  return hipGetLastError();
}

}  // namespace sage
