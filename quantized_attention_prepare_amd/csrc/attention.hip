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
// Schedule (per wave, iteration t: a fixed sequence of slots, one MFMA each)
//   the FP8 PV MFMAs of tile t-1 issue under the maximum of tile t's scores
//   and its first exp2 / FP8 groups; then the INT8 score MFMAs of tile t+1
//   (not needed before the next iteration) issue under the remaining exp2
//   groups, the update of l and the rescale of O. The matrix cores thus work
//   under the same wave's softmax; the other workgroup on the CU,
//   unsynchronised with this one, fills the remaining gaps. Causal attention
//   stops at the key tile of the workgroup's own queries and masks it per lane.
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
// Head dims 128 and 64 share this code (template parameter D): D/32 score
// MFMA steps per 32-key block, D/32 output channel blocks; the key tile stays
// 128 (it is part of the result's definition).
//
// LDS (5 * 128 * D bytes per workgroup: 80 KB at D = 128): two K tiles
// [128 keys][D B] and two V tiles [D ch][128 B] (tile t in buffer t & 1),
// filled by buffer loads that write LDS directly, and the workgroup's 128 INT8
// query rows. During iteration t the wave reads K(t+1) and V(t-1) while K(t+2)
// and V(t) are being copied.
// Bank layout: gfx950 serves a ds_read_b128 16 lanes at a time from 64 banks of
// 4 bytes, so 16 consecutive lanes must hit 16 different 16-byte slots of a
// 256-byte bank row. The 16-byte chunk c of row r is stored at c XOR f(r).
// 128-byte rows (two per bank row; V always, K and Q at D = 128): for V and Q
// f(r) = (r>>1)&7, for K, whose rows are read in the permuted order pi,
// f(r) = ((r>>1)&3) | ((r>>4)&1)<<2. 64-byte rows (four per bank row; K and Q
// at D = 64): for Q f(r) = (r>>2)&3, for K f(r) = ((r>>2)&1) | ((r>>4)&1)<<1.
#include "prologue_ops.hpp"

namespace sage {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPerWg = 32 * kWaves;

// Geometry of one head dim D.
template <int D>
struct Dim {
  static constexpr int kTileBytes = kKvTile * D;            // one K or V tile
  static constexpr int kCopyInstr = kTileBytes / 1024 / kWaves;   // 1 KB copy instructions per wave per tile
  static constexpr int kSteps = D / 32;                     // 32-channel steps of a score MFMA chain
  static constexpr int kOBlk = D / 32;                      // 32-channel output blocks
  static constexpr int kChunks = D / 16;                    // 16-byte chunks in a K or Q row
  // LDS swizzles (see the header): K rows read in the order pi, Q rows by query
  static __device__ int fk(int r) {
    return D == 128 ? (((r >> 1) & 3) | (((r >> 4) & 1) << 2)) : (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
  }
  static __device__ int fq(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
};
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448): folds the P scale into exp2
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kBufferWord3 = 0x00020000;          // raw (untyped) buffer access

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#define SAGE_INLINE __device__ __attribute__((always_inline)) inline

// Global -> LDS copies with buffer loads that write LDS directly (16 B per
// lane). Each wave moves a quarter of a tile: instruction i of wave w fills the
// j-th KB of the tile, j = kCopyInstr w + i, lane t landing at byte 16 t of
// it. The lane fetches the global chunk that belongs at its swizzled position,
// which depends only on the lane and on j, so each instruction's lane offset
// is a per-lane constant. One buffer resource per head holds the 64-bit base
// and the exact byte extent (the hardware bounds-checks every copy); tile and
// row offsets go in the 32-bit scalar offset and the lane offset in one vector
// register.
// K tile t: 128 keys x D B, contiguous in k8 (head extent S_pad * D B).
// The LDS destination goes through an empty asm so that its per-instruction
// addresses are formed next to each copy instead of being precomputed for
// every buffer and kept live in scalar registers across the loop.
SAGE_INLINE uint8_t* opaque_lds(uint8_t* dst) {
  uint32_t a = (uint32_t)(uintptr_t)LDS_PTR(dst);
  asm volatile("" : "+s"(a));
  return (uint8_t*)(__attribute__((address_space(3))) uint8_t*)(uintptr_t)a;
}
template <int D>
SAGE_INLINE void load_k(uint8_t* dst, __amdgpu_buffer_rsrc_t rk, int t, const uint32_t* lane_off, int wave) {
  constexpr int C = Dim<D>::kCopyInstr;
  dst = opaque_lds(dst);
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass has no LDS-destination buffer load
#pragma unroll
  for (int i = 0; i < C; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS_PTR(dst + 1024 * (C * wave + i)), 16, lane_off[i],
                                             (uint32_t)t * Dim<D>::kTileBytes + 1024u * (C * wave + i), 0, 0);
#endif
}
// V tile t: D channels x 128 keys; channel rows are S_pad bytes apart in v8t
// (head extent D * S_pad B); each KB is 8 channel rows.
template <int D>
SAGE_INLINE void load_v(uint8_t* dst, __amdgpu_buffer_rsrc_t rv, int t, uint32_t S_pad, const uint32_t* lane_off,
                        int wave) {
  constexpr int C = Dim<D>::kCopyInstr;
  dst = opaque_lds(dst);
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
  for (int i = 0; i < C; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, LDS_PTR(dst + 1024 * (C * wave + i)), 16, lane_off[i],
                                             (uint32_t)t * kKvTile + (uint32_t)(8 * (C * wave + i)) * S_pad, 0, 0);
#endif
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
template <int D>
struct WaveState {
  v16f oacc[D / 32];   // O^T blocks: channels 32*d + 8(v/4) + 4h + v%4 of this lane's query
  v8i pk[2];      // FP8 probabilities of the tile whose PV is next (two 64-key halves)
  float m_run;    // running max (log2 units)
  float l_run;    // this lane-half's share of 448 * sum p
};

// INT8 scores S^T = K . Q^T of one tile into sacc: row pi(col) of each 32-key
// block, channels 32s + 16h .. +15; the four score blocks are independent
// MFMAs.
template <int D>
SAGE_INLINE void qk_tile(v16i (&sacc)[4], const uint8_t* kbuf, const uint8_t* qrow, int half, int col, int prow) {
  const uint8_t* krow = kbuf + prow * D;
  const int fk = Dim<D>::fk(prow);   // f(32 kb + prow) for every kb
  const int fq = Dim<D>::fq(col);
#pragma unroll
  for (int s = 0; s < Dim<D>::kSteps; ++s) {
    const v4i qb = *reinterpret_cast<const v4i*>(qrow + (((2 * s + half) ^ fq) * 16));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const v4i a = *reinterpret_cast<const v4i*>(krow + 32 * kb * D + (((2 * s + half) ^ fk) * 16));
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
// rescale of O; the next tile's scores go to snext.
// cblk[kb] = (q_scale * k_scale) * sm_scale * log2 e of the tile's 32-key
// blocks. nvalid < 128 marks a ragged last tile: the padded keys' scores are
// replaced with INT32_MIN (never above a valid score since |acc| <= 2^21),
// blocks made only of padding come with cblk = +inf (probability exactly 0),
// and in the partly padded block the padded keys' probability, which only
// matters for l (their V codes are 0), is subtracted from l afterwards.
SAGE_INLINE int max3i(int a, int b, int c) { return max(max(a, b), c); }

#define SAGE_FENCE() __builtin_amdgcn_sched_barrier(0)

// V^T operand of PV MFMA (kc, d): channel 32d + col, keys 64kc + 32(j/16) + 16h + j%16.
SAGE_INLINE v8i v_operand(const uint8_t* vbuf, int kc, int d, int half, int col, int fv) {
  const uint8_t* vrow = vbuf + (32 * d + col) * kKvTile;
  union { v8i v; v4i q[2]; } a;
  a.q[0] = *reinterpret_cast<const v4i*>(vrow + (((4 * kc + half) ^ fv) * 16));
  a.q[1] = *reinterpret_cast<const v4i*>(vrow + (((4 * kc + 2 + half) ^ fv) * 16));
  return a.v;
}

// Max of t = float(acc) * c over the lane's 16 keys of one 32-key block: a
// tree of three-input maxima on the integer accumulators; float(max acc) * c
// is the max of the products because c >= 0 and rounding is monotone.
SAGE_INLINE float block_max(const v16i& x, float c) {
  const int a0 = max3i(x[0], x[1], x[2]), a1 = max3i(x[3], x[4], x[5]), a2 = max3i(x[6], x[7], x[8]);
  const int a3 = max3i(x[9], x[10], x[11]), a4 = max3i(x[12], x[13], x[14]);
  const int im = max(max3i(a0, a1, a2), max3i(a3, a4, x[15]));
  return (float)im * c;
}

// Probabilities of 4 consecutive keys (group g of block kb), 448 p for the
// score t = float(acc) * c, summed into ps, packed to FP8 into pk.
// Fast form (kExact false, moff = m' - log2 448): 448 p = exp2(acc c - moff) in
// one FMA, without the method's rounding of t to float first. That rounding
// moves the exponent by at most half an ulp of t: negligible while |t| is
// moderate, whole units once |t| passes 2^24, where the FMA form can even
// exceed 448 (an FP8 NaN). Waves whose scores may reach 2^14 in magnitude
// therefore take the exact form (kExact true, moff = m'): the method's own
// steps, p = exp2(t - m') with t rounded to float first, then 448 p.
template <bool kExact, bool kFirst = false>
SAGE_INLINE void exp_group(const v16i& sc, int kb, int g, float c, float moff, v8i (&pk)[2], float (&ps)[4]) {
  float p[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if constexpr (kExact)   // a product, then a difference: no contraction (-ffp-contract=off)
      p[u] = 448.0f * __builtin_amdgcn_exp2f((float)sc[4 * g + u] * c - moff);
    else
      p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)sc[4 * g + u], c, -moff));
    if constexpr (kFirst)   // the tile's first group starts the partial sums (0 + p would cost an add)
      ps[u] = p[u];
    else
      ps[u] += p[u];
  }
  const int j = 16 * (kb & 1) + 4 * g;   // k-slot of p[0] within the 64-key half-tile
  // the first conversion writes bytes 0-1 and the second bytes 2-3, so the word
  // they start from does not matter: p[0]'s own register serves (0 would cost
  // a move per word)
  int dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
  dw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], dw, true);
  // keep the packing in its slot: left free, the compiler sinks the packs of
  // one of the two unrolled tiles past the rescale branch into the loop
  // latch, which keeps that tile's 64 float probabilities live across the
  // branch (about 40 more VGPRs)
  asm volatile("" ::"v"(dw));
  pk[kb >> 1][j >> 2] = dw;
}

// One iteration, as a fixed sequence of slots separated by scheduling fences,
// each slot holding at most one MFMA and a run of VALU work that issues while
// the MFMA executes:
//   slots 1-8   PV of the previous tile (its probabilities in pk, its V tile in
//               vbuf_prev), with the maximum of this tile's scores (one block
//               per slot) and then the exp2 of blocks 0 and 1 (whose FP8 codes
//               go to pk[0] once the MFMAs that read the previous pk[0] have
//               been issued);
//   slots 9-24  the INT8 score MFMAs of the next tile, with the exp2 of blocks
//               2 and 3, l, and the rescale of O (the previous PV is complete by
//               then).
// At D = 64 there are four PV and eight score MFMAs, two exp2 groups per slot.
// The LDS operands of each MFMA are read two slots ahead. kHasPrev is false for
// the first tile. cblk[kb] = (q_scale * k_scale) * sm_scale * log2 e of the
// tile's 32-key blocks. nvalid < 128 marks a ragged last tile: padded keys'
// scores become INT32_MIN (below every valid score since |acc| <= 2^21), blocks
// made only of padding come with cblk = +inf (probability exactly 0), and in
// the partly padded block the padded keys' probability, which only matters for
// l (their V codes are 0), is subtracted from l afterwards.
// In general a masked tile (masked = true) gives each lane its own limit lim:
// the lane sees the tile's keys below lim. Causal attention's diagonal tile
// uses lim = min(query + 1, nvalid) (tile-relative), with cblk = +inf for the
// blocks no lane of the wave sees; each lane then has at most one partly
// masked block, whose masked keys' probability comes off l as above. Their
// FP8 codes, which meet real V codes there, are cleared before that tile's PV.
template <int D, bool kHasPrev, bool kExact>
SAGE_INLINE void tile_iteration(WaveState<D>& st, v16i (&sc)[4], v16i (&snext)[4], const float (&cblk)[4],
                                bool masked, int lim, const uint8_t* vbuf_prev, const uint8_t* kbuf_next,
                                const uint8_t* qrow, int half, int col, int prow) {
  const int kbase = 16 * half;
  const int fk = Dim<D>::fk(prow);   // K swizzle of rows 32 kb + prow
  const int fq = Dim<D>::fq(col);    // Q swizzle of row col
  const int fv = (col >> 1) & 7;     // V swizzle of rows 32 d + col
  const uint8_t* krow = kbuf_next + prow * D;
  // ---- slot 0: first two V operands; tail masking; max of block 0
  // Operands are read two slots ahead into alternating registers (one slot of
  // VALU work is often shorter than an LDS read): PV MFMA P reads vv[P & 1],
  // score MFMA Q reads kk[Q & 1] and qq[(Q / 4) & 1].
  constexpr int NPV = 2 * Dim<D>::kOBlk;          // PV MFMAs (kc outer, d inner)
  constexpr int NQK = 4 * Dim<D>::kSteps;         // score MFMAs (s outer, kb inner)
  v8i vv[2];
  v4i kk[2], qq[2];
  if (kHasPrev) {
    vv[0] = v_operand(vbuf_prev, 0, 0, half, col, fv);
    vv[1] = v_operand(vbuf_prev, 1 / Dim<D>::kOBlk, 1 % Dim<D>::kOBlk, half, col, fv);
  }
  if (masked) {
    // Only the last tile gets here. The empty asm hides that nvalid is then
    // the loop-invariant length of the last tile, which would otherwise move
    // the 64 key-index comparisons out of the loop into live lane masks; the
    // selection uses sign masks rather than comparisons for the same reason.
    int nv = lim - kbase;
    asm volatile("" : "+v"(nv));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int keep = (32 * kb + v - nv) >> 31;   // all ones for a valid key
        sc[kb][v] = (sc[kb][v] & keep) | (INT32_MIN & ~keep);
      }
  }
  float tmax = block_max(sc[0], cblk[0]);
  SAGE_FENCE();
#define SAGE_KOP(Q_) (*reinterpret_cast<const v4i*>(krow + 32 * ((Q_) % 4) * D + (((2 * ((Q_) / 4) + half) ^ fk) * 16)))
#define SAGE_QOP(S_) (*reinterpret_cast<const v4i*>(qrow + (((2 * (S_) + half) ^ fq) * 16)))
#define SAGE_PV_SLOT(P_, WORK_)                                                                              \
  {                                                                                                           \
    if (kHasPrev) {                                                                                           \
      constexpr int kc_ = (P_) / Dim<D>::kOBlk, d_ = (P_) % Dim<D>::kOBlk;                                    \
      st.oacc[d_] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vv[(P_) & 1], st.pk[kc_], st.oacc[d_], 0, \
                                                                    0, 0, 0, 0, 0);                           \
      if ((P_) + 2 < NPV)                                                                                     \
        vv[(P_) & 1] = v_operand(vbuf_prev, ((P_) + 2) / Dim<D>::kOBlk, ((P_) + 2) % Dim<D>::kOBlk, half, col, \
                                 fv);                                                                         \
    }                                                                                                         \
    if ((P_) == NPV - 2) {                                                                                    \
      qq[0] = SAGE_QOP(0);                                                                                    \
      kk[0] = SAGE_KOP(0);                                                                                    \
    }                                                                                                         \
    if ((P_) == NPV - 1) kk[1] = SAGE_KOP(1);                                                                 \
    WORK_;                                                                                                    \
    SAGE_FENCE();                                                                                             \
  }
  float m_new, alpha, moff;
  float ps[4];
#define SAGE_EXP(KB_, G_) exp_group<kExact, (KB_) == 0 && (G_) == 0>(sc[KB_], KB_, G_, cblk[KB_], moff, st.pk, ps)
#define SAGE_L_UPDATE()                                                                               \
  {                                                                                                   \
    float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);                                                   \
    if (masked && (lim & 31)) {                                                                       \
      const int kbp = lim >> 5; /* the partly masked block */                                         \
      const int nmask = min(16, max(0, 32 * kbp + kbase + 16 - lim));                                 \
      const float ck = cblk[kbp];                                                                     \
      const float pm = kExact ? 448.0f * __builtin_amdgcn_exp2f((float)INT32_MIN * ck - moff)         \
                              : __builtin_amdgcn_exp2f(__builtin_fmaf((float)INT32_MIN, ck, -moff));  \
      if (nmask > 0) psum -= (float)nmask * pm;                                                       \
    }                                                                                                 \
    st.l_run = alpha * st.l_run + psum;                                                               \
    st.m_run = m_new;                                                                                 \
  }
  if constexpr (D == 128) {
  SAGE_PV_SLOT(0, tmax = fmaxf(tmax, block_max(sc[1], cblk[1])))
  SAGE_PV_SLOT(1, tmax = fmaxf(tmax, block_max(sc[2], cblk[2])))
  SAGE_PV_SLOT(2, tmax = fmaxf(tmax, block_max(sc[3], cblk[3])))
  SAGE_PV_SLOT(3, {
    tmax = max_xor32(tmax);
    m_new = fmaxf(st.m_run, tmax);
    alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 0 on the first tile
    moff = kExact ? m_new : m_new - kLog2_448;          // see exp_group
  })
  // pk[0] of the previous tile has been handed to its MFMAs: blocks 0, 1 may overwrite it
  SAGE_PV_SLOT(4, { SAGE_EXP(0, 0); SAGE_EXP(0, 1); })
  SAGE_PV_SLOT(5, { SAGE_EXP(0, 2); SAGE_EXP(0, 3); })
  SAGE_PV_SLOT(6, { SAGE_EXP(1, 0); SAGE_EXP(1, 1); })
  SAGE_PV_SLOT(7, { SAGE_EXP(1, 2); SAGE_EXP(1, 3); })
  } else {
  SAGE_PV_SLOT(0, tmax = fmaxf(tmax, fmaxf(block_max(sc[1], cblk[1]), block_max(sc[2], cblk[2]))))
  SAGE_PV_SLOT(1, {
    tmax = fmaxf(tmax, block_max(sc[3], cblk[3]));
    tmax = max_xor32(tmax);
    m_new = fmaxf(st.m_run, tmax);
    alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);   // 0 on the first tile
    moff = kExact ? m_new : m_new - kLog2_448;          // see exp_group
  })
  // pk[0] of the previous tile has been handed to its MFMAs: blocks 0, 1 may overwrite it
  SAGE_PV_SLOT(2, { SAGE_EXP(0, 0); SAGE_EXP(0, 1); })
  SAGE_PV_SLOT(3, { SAGE_EXP(0, 2); SAGE_EXP(0, 3); })
  }
#undef SAGE_PV_SLOT
  // ---- score MFMAs of the next tile (s outer, kb inner)
#define SAGE_QK_SLOT(Q_, WORK_)                                                                          \
  {                                                                                                       \
    constexpr int s_ = (Q_) / 4, kb_ = (Q_) % 4;                                                          \
    const v16i z = {};                                                                                    \
    snext[kb_] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kk[(Q_) & 1], qq[s_ & 1], s_ == 0 ? z : snext[kb_], 0, \
                                                       0, 0);                                             \
    if ((Q_) + 2 < NQK) {                                                                                 \
      if (((Q_) + 2) % 4 == 0) qq[(((Q_) + 2) / 4) & 1] = SAGE_QOP(((Q_) + 2) / 4);                       \
      kk[(Q_) & 1] = SAGE_KOP((Q_) + 2);                                                                  \
    }                                                                                                     \
    WORK_;                                                                                                \
    SAGE_FENCE();                                                                                         \
  }
  if constexpr (D == 128) {
  SAGE_QK_SLOT(0, SAGE_EXP(2, 0))
  SAGE_QK_SLOT(1, (void)0)
  SAGE_QK_SLOT(2, SAGE_EXP(2, 1))
  SAGE_QK_SLOT(3, (void)0)
  SAGE_QK_SLOT(4, SAGE_EXP(2, 2))
  SAGE_QK_SLOT(5, (void)0)
  SAGE_QK_SLOT(6, SAGE_EXP(2, 3))
  SAGE_QK_SLOT(7, (void)0)
  SAGE_QK_SLOT(8, SAGE_EXP(3, 0))
  SAGE_QK_SLOT(9, (void)0)
  SAGE_QK_SLOT(10, SAGE_EXP(3, 1))
  SAGE_QK_SLOT(11, (void)0)
  SAGE_QK_SLOT(12, SAGE_EXP(3, 2))
  SAGE_QK_SLOT(13, (void)0)
  SAGE_QK_SLOT(14, SAGE_EXP(3, 3))
  SAGE_QK_SLOT(15, SAGE_L_UPDATE())
  } else {
  SAGE_QK_SLOT(0, { SAGE_EXP(1, 0); SAGE_EXP(1, 1); })
  SAGE_QK_SLOT(1, { SAGE_EXP(1, 2); SAGE_EXP(1, 3); })
  // pk[1] of the previous tile has been handed to its MFMAs as well
  SAGE_QK_SLOT(2, { SAGE_EXP(2, 0); SAGE_EXP(2, 1); })
  SAGE_QK_SLOT(3, { SAGE_EXP(2, 2); SAGE_EXP(2, 3); })
  SAGE_QK_SLOT(4, { SAGE_EXP(3, 0); SAGE_EXP(3, 1); })
  SAGE_QK_SLOT(5, { SAGE_EXP(3, 2); SAGE_EXP(3, 3); })
  SAGE_QK_SLOT(6, SAGE_L_UPDATE())
  SAGE_QK_SLOT(7, (void)0)
  }
#undef SAGE_L_UPDATE
#undef SAGE_QK_SLOT
#undef SAGE_KOP
#undef SAGE_QOP
#undef SAGE_EXP
  // Rescale O to the new maximum (the previous tile's PV has completed by
  // now), only when some lane's maximum moved: alpha exactly 1 multiplies by
  // one, and after the first tiles that is the usual case.
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int d = 0; d < Dim<D>::kOBlk; ++d)
#pragma unroll
      for (int v = 0; v < 16; ++v) st.oacc[d][v] *= alpha;
  }
}

// PV of the last tile, after the loop.
template <int D>
SAGE_INLINE void pv_tile(WaveState<D>& st, const uint8_t* vbuf, int half, int col) {
  const int fv = (col >> 1) & 7;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int d = 0; d < Dim<D>::kOBlk; ++d)
      st.oacc[d] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v_operand(vbuf, kc, d, half, col, fv), st.pk[kc],
                                                                   st.oacc[d], 0, 0, 0, 0, 0, 0);
}

// The key loop of one wave, its tail and the epilogue: the online softmax
// state starts here, so the two copies (fast and exact form) share no state
// and are register-allocated independently.
// kResident: every K tile of the head is in LDS from lds on (tile t at
// lds + t TB) and every V tile from vres on, in the layout the copies give
// them; the loop then copies nothing and passes no barrier, so the waves of a
// workgroup may run different numbers of tiles. v_scale then points at the
// head's D scales themselves.
template <int D, bool kCausal, bool kExact, bool kResident = false>
SAGE_INLINE void key_loop(uint8_t* lds, uint8_t* vres, __amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                          const uint32_t (&k_lane_off)[Dim<D>::kCopyInstr],
                          const uint32_t (&v_lane_off)[Dim<D>::kCopyInstr], const float* ks, float qs, float sl2,
                          const uint8_t* qrow, int prow, int wave, int half, int col, int ntw, int ntiles,
                          int last_valid, uint32_t spad32, int64_t q0, int64_t S, int64_t bh, int64_t b, int64_t h,
                          const float* __restrict__ v_scale, const Bf16OutView& o, float* __restrict__ lse) {
  using Dm = Dim<D>;
  constexpr int TB = Dm::kTileBytes;
  // q_scale * (sm_scale * log2 e): the fast form's block constant is this times
  // k_scale, one product per block (an ulp away from the method's
  // (q_scale * k_scale) * (sm_scale * log2 e), well inside the fast form's
  // other differences)
  const float qsl2 = qs * sl2;
#define KBUF(i) (lds + (i) * TB)
#define VBUF(i) (lds + (2 + (i)) * TB)
  WaveState<D> st;
#pragma unroll
  for (int d = 0; d < Dm::kOBlk; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) st.oacc[d][v] = 0.0f;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc)
#pragma unroll
    for (int i = 0; i < 8; ++i) st.pk[kc][i] = 0;
  st.m_run = -INFINITY;
  st.l_run = 0.0f;

  v16i sa[4], sb[4];   // scores of the current and the next tile; they swap roles every iteration
  qk_tile<D>(sa, KBUF(0), qrow, half, col, prow);
  float4 ksv = *reinterpret_cast<const float4*>(ks);   // k_scale of the four blocks of the current tile

  // Iteration t: PV of tile t-1, softmax of tile t, scores of tile t+1. On
  // entry K(t+1) and V(t-1) must be in LDS; K(t+2) goes to the buffer K(t)
  // occupied and V(t) to the one V(t-2) occupied. After the last tile the
  // score MFMAs read stale K bytes whose scores are never used.
  // Causal: the last visited tile holds the workgroup's own queries; there
  // the lane sees keys below min(32 wave + col + 1, nvalid), and blocks at or
  // past min(32 (wave + 1), nvalid) are masked for the whole wave.
#define SAGE_ITERATION(T_, PAR_, HAS_PREV_, CUR_, NEXT_)                                                     \
  {                                                                                                          \
    const int t_ = (T_);                                                                                     \
    if constexpr (!kResident) {                                                                              \
      __builtin_amdgcn_s_waitcnt(0); /* this wave's copies have landed */                                    \
      __syncthreads();               /* ... everyone's; K(t) and V(t-2) are no longer read */                \
      if (t_ + 2 < ntw) load_k<D>(KBUF(PAR_), rk, t_ + 2, k_lane_off, wave);                                 \
      load_v<D>(VBUF(PAR_), rv, t_, spad32, v_lane_off, wave);                                               \
    }                                                                                                        \
    const int nvalid = t_ == ntiles - 1 ? last_valid : kKvTile;                                              \
    const bool diag = kCausal && t_ == ntw - 1;                                                              \
    const int nblk = diag ? min(32 * (wave + 1), nvalid) : nvalid;                                           \
    const float kss[4] = {ksv.x, ksv.y, ksv.z, ksv.w};                                                       \
    /* q_scale * k_scale * sm_scale * log2 e (the exact form: the method's product order); */                \
    /* +inf for a block masked for the whole wave, which only masked tiles have */                           \
    float cblk[4];                                                                                           \
    for (int kb = 0; kb < 4; ++kb) cblk[kb] = kExact ? (qs * kss[kb]) * sl2 : qsl2 * kss[kb];                \
    if (diag || nvalid < kKvTile)                                                                            \
      for (int kb = 0; kb < 4; ++kb) cblk[kb] = 32 * kb >= nblk ? INFINITY : cblk[kb];                       \
    if (t_ + 1 < ntw) ksv = *reinterpret_cast<const float4*>(ks + 4 * (t_ + 1));                             \
    tile_iteration<D, HAS_PREV_, kExact>(st, CUR_, NEXT_, cblk, diag || nvalid < kKvTile,                    \
                                         diag ? min(32 * wave + col + 1, nvalid) : nvalid,                   \
                                         kResident ? vres + (t_ - 1) * TB : VBUF((PAR_) ^ 1),                \
                                         kResident ? lds + (t_ + 1) * TB : KBUF((PAR_) ^ 1), qrow, half, col, \
                                         prow);                                                              \
  }
  // tile t uses buffer pair t & 1; the parity is spelled out so that buffer
  // addresses fold into the LDS instructions' offsets (t is odd in the loop)
  SAGE_ITERATION(0, 0, false, sa, sb)
  int t = 1;
  for (; t + 1 < ntw; t += 2) {
    SAGE_ITERATION(t, 1, true, sb, sa)
    SAGE_ITERATION(t + 1, 0, true, sa, sb)
  }
  if (t < ntw) SAGE_ITERATION(t, 1, true, sb, sa)
#undef SAGE_ITERATION
  if constexpr (kCausal) {
    // Clear the FP8 codes of the diagonal tile's masked keys (those at or past
    // lim), whose V codes are real: byte u of pk[kc][i] is key
    // 32 kb + 16 half + 4 g + u of the tile, kb = 2 kc + i / 4, g = i % 4.
    const int lim = min(32 * wave + col + 1, ntw == ntiles ? last_valid : kKvTile);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int base = 32 * (2 * kc + i / 4) + 16 * half + 4 * (i % 4);
        const int nb = min(4, max(0, lim - base));   // valid bytes of the word
        const uint32_t keep = nb == 4 ? 0xFFFFFFFFu : (1u << (8 * nb)) - 1u;
        st.pk[kc][i] &= (int)keep;
      }
  }
  // PV of the last tile
  if constexpr (!kResident) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  pv_tile<D>(st, kResident ? vres + (ntw - 1) * TB : VBUF((ntw - 1) & 1), half, col);

  // ---- epilogue: O = o * v_scale / (448 l)
  const float l_tot = st.l_run + __shfl_xor(st.l_run, 32, 64);
  const float inv_l = 1.0f / l_tot;
  const int64_t qi = q0 + col;
  // log-sum-exp of the row's dequantized scores, natural log: l_tot = 448 sum_j 2^(t_j - m)
  if (lse != nullptr && half == 0 && qi < S) lse[bh * S + qi] = (st.m_run + __log2f(l_tot) - kLog2_448) * kLn2;
  if (qi < S) {
    uint16_t* orow = o.data + b * o.sb + qi * o.ss + h * o.sh;
    const float* vs = kResident ? v_scale : v_scale + bh * D;   // resident: the head's own scales
#pragma unroll
    for (int d = 0; d < Dm::kOBlk; ++d) {
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

template <int D, bool kCausal>
__global__ void __launch_bounds__(kThreads, 2)
attn_kernel(const int8_t* __restrict__ q8, const float* __restrict__ q_scale, const int8_t* __restrict__ k8,
            const float* __restrict__ k_scale, const uint8_t* __restrict__ v8t, const float* __restrict__ v_scale,
            int64_t H, int64_t S, int64_t S_pad, int64_t nqt, int64_t nwg, float sl2, Bf16OutView o,
            float* __restrict__ lse) {
  using Dm = Dim<D>;
  constexpr int C = Dm::kCopyInstr, TB = Dm::kTileBytes;
  // two K and two V tile buffers (indexed by tile & 1), then the workgroup's
  // 128 query rows [query][D B] (16-byte chunks XOR swizzled by fq(query))
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TB + kQPerWg * D];
#define KBUF(i) (lds + (i) * TB)
#define VBUF(i) (lds + (2 + (i)) * TB)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  // K copy: the j-th KB (j = C wave + i) holds rows (1024 / D) j + lane / (D/16),
  // lane landing at chunk lane % (D/16); it fetches global chunk
  // (lane % (D/16)) XOR fk(row)
  uint32_t k_lane_off[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int j = C * wave + i;
    const int row = (1024 / D) * j + lane / Dm::kChunks, slot = lane % Dm::kChunks;
    k_lane_off[i] = (uint32_t)((lane / Dm::kChunks) * D + ((slot ^ Dm::fk(row)) * 16));
  }

  // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs;
  // give each XCD a contiguous range of (head, query tile) so the query tiles
  // of one head share that XCD's L2 while they stream the same K/V.
  const int64_t bid = blockIdx.x;
  const int64_t per = nwg / 8, rem = nwg % 8, x = bid % 8;
  const int64_t logical = x * per + (x < rem ? x : rem) + bid / 8;
  int64_t bh = logical / nqt;
  int64_t qt = logical % nqt;
  if (kCausal) {
    // Causal: query tile qt costs qt + 1 key tiles. Workgroups go out longest
    // first (every head's last query tile, then the one before, ...), so the
    // short tiles fill in at the end, and each XCD receives every eighth of
    // them, a balanced share. Consecutive query tiles of one head are B*H
    // workgroups apart: with B*H = 4 (mod 8), as for 28 heads, a head's tiles
    // alternate between two XCDs.
    const int64_t nbh = nwg / nqt;
    qt = nqt - 1 - bid / nbh;
    bh = bid % nbh;
  }
  const int64_t b = bh / H, h = bh % H;

  const int64_t q0 = qt * kQPerWg + 32 * wave;   // this wave's first query (one INT8 block)
  const bool active = q0 < S_pad;                // the last workgroup may reach past S_pad
  const uint32_t spad32 = (uint32_t)S_pad;       // 128 S_pad < 2^32 (host check)
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k8 + bh * S_pad * D), 0, (int)(spad32 * D), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v8t + bh * D * S_pad), 0, (int)(spad32 * D), kBufferWord3);
  // V copy: the j-th KB holds channel rows 8 j + lane / 8 (128 B each); the
  // swizzle (row >> 1) & 7 = ((lane >> 4) & 3) | ((j & 1) << 2), and j & 1 =
  // i & 1 because C is even
  static_assert(C % 2 == 0, "V copy swizzle assumes an even number of copies per wave");
  uint32_t v_lane_off[C];
#pragma unroll
  for (int i = 0; i < C; ++i)
    v_lane_off[i] = (uint32_t)(lane >> 3) * spad32 + (uint32_t)(((lane & 7) ^ (((lane >> 4) & 3) | ((i & 1) << 2))) * 16);
  const float* ks = k_scale + bh * (S_pad / kQBlock);
  float qs = active ? q_scale[bh * (S_pad / kQBlock) + q0 / kQBlock] : 0.0f;
  // Key-block scale from which this wave's scores may reach 2^14 in magnitude
  // (|acc| <= 128 * 127^2 < 2^21), as float bits (scales are >= 0, so their
  // bits order like their values). Ordinary inputs stay far below it (scores of
  // tens); q_scale 0 gives +inf (never reached).
  const uint32_t kexact = __builtin_amdgcn_readfirstlane(__float_as_uint(0x1p-7f / (sl2 * qs)));
  // kept in a vector register: a VALU operation reads at most one scalar
  // register, and the key-block scales arrive in scalar registers
  asm volatile("" : "+v"(qs));

  // This wave's 32 query rows go to LDS once (zeros past S_pad); the score
  // MFMAs read their B operand from there.
  uint8_t* qlds = lds + 4 * TB + 32 * wave * D;
  {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      // row r of the wave, 16-byte chunk c
      const int r = (1024 / D) * i + lane / Dm::kChunks, c = lane % Dm::kChunks;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (active) val = *reinterpret_cast<const uint4*>(q8 + (bh * S_pad + q0 + r) * D + c * 16);
      *reinterpret_cast<uint4*>(qlds + r * D + ((c ^ Dm::fq(r)) * 16)) = val;
    }
  }
  const uint8_t* qrow = qlds + col * D;
  // A-operand row of the score MFMA fed by this lane: key pi(col) of a 32-key block
  const int prow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  const int ntiles = (int)(S_pad / kKvTile);
  const int last_valid = (int)(S - (int64_t)(ntiles - 1) * kKvTile);   // valid keys in the last tile (1..128)
  // key tiles this workgroup visits: causal stops at the tile of its own
  // queries (a query tile is one key tile: 128 rows)
  static_assert(kQPerWg == kKvTile, "causal tiling assumes query tile = key tile");
  const int ntw = kCausal ? (int)qt + 1 : ntiles;

  // K(0), K(1) in; scores of tile 0.
  load_k<D>(KBUF(0), rk, 0, k_lane_off, wave);
  if (ntw > 1) load_k<D>(KBUF(1), rk, 1, k_lane_off, wave);
  // The largest key-block scale this wave meets (bits; scales are >= 0), read
  // while the tiles load: at or above kexact the wave runs the exact form of
  // the softmax step (see exp_group) in its own copy of the key loop. The two
  // copies pass the same barriers, so the waves of a workgroup may differ.
  uint32_t kmax = 0;
  for (int i = lane; i < 4 * ntw; i += 64) kmax = max(kmax, __float_as_uint(ks[i]));
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (__builtin_expect(__builtin_amdgcn_readfirstlane(kmax) >= kexact, 0)) {
    key_loop<D, kCausal, true>(lds, nullptr, rk, rv, k_lane_off, v_lane_off, ks, qs, sl2, qrow, prow, wave, half, col, ntw,
                               ntiles, last_valid, spad32, q0, S, bh, b, h, v_scale, o, lse);
    return;
  }
  key_loop<D, kCausal, false>(lds, nullptr, rk, rv, k_lane_off, v_lane_off, ks, qs, sl2, qrow, prow, wave, half, col, ntw,
                              ntiles, last_valid, spad32, q0, S, bh, b, h, v_scale, o, lse);
#undef KBUF
#undef VBUF
}


// ------------------------------------------------------------- short heads
// A head of at most Short<D>::kTiles key tiles is handled start to end by one
// workgroup of kShortWaves waves, in one launch: first the prologue's steps for
// the head, with the arithmetic of its three passes (the same codes and
// scales), every code and scale kept in LDS (K and V codes in the layout the
// tile copies above give them, Q codes in the layout of the query rows); then
// each wave runs the key loop over the resident tiles for its 32-query blocks.
// The statistics pass is split into pieces (one tensor of one 32-row block)
// handed to the waves in turn, so they share them evenly. At head dim 64 a
// wave loads its next piece while it works on the current one and keeps every
// V block it read in registers until the V codes can be formed; at head dim
// 128, where registers are scarcer, it keeps its first V block and reads any
// other one again.
constexpr int kShortWaves = 8;
template <int D>
struct Short {
  static constexpr int kTiles = D == 128 ? 3 : 6;   // resident K, V and Q that fit in LDS
  static constexpr int kBlocks = 4 * kTiles;        // 32-row blocks
  static constexpr int kVPerWave = (kBlocks + kShortWaves - 1) / kShortWaves;   // V blocks a wave reads
  static constexpr int kVKept = D == 128 ? 1 : kVPerWave;   // of them held in registers (the rest read again)
};

// Codes of rows 32 (j % 4) + G i + g of K tile j / 4 (channels 8c..8c+7 in
// lo[i], hi[i]) into the resident tile: chunk (c / 2) of row r sits at slot
// (c / 2) XOR fk(r).
template <int D>
SAGE_INLINE void put_k_rows(uint8_t* kres, int j, const uint32_t (&lo)[Geo<D>::I], const uint32_t (&hi)[Geo<D>::I],
                            int c, int g) {
  using Gm = Geo<D>;
  uint8_t* tile = kres + (j >> 2) * Dim<D>::kTileBytes;
#pragma unroll
  for (int i = 0; i < Gm::I; ++i) {
    const int r = 32 * (j & 3) + Gm::G * i + g;
    *reinterpret_cast<uint2*>(tile + r * D + ((((c >> 1) ^ Dim<D>::fk(r)) << 4) | ((c & 1) << 3))) =
        make_uint2(lo[i], hi[i]);
  }
}

// Codes of query block j into its 32 resident rows: chunk (c / 2) of row r at
// slot (c / 2) XOR fq(r), as the attention kernel stores its query rows.
template <int D>
SAGE_INLINE void put_q_rows(uint8_t* qblk, const uint32_t (&lo)[Geo<D>::I], const uint32_t (&hi)[Geo<D>::I], int c,
                            int g) {
  using Gm = Geo<D>;
#pragma unroll
  for (int i = 0; i < Gm::I; ++i) {
    const int r = Gm::G * i + g;
    *reinterpret_cast<uint2*>(qblk + r * D + ((((c >> 1) ^ Dim<D>::fq(r)) << 4) | ((c & 1) << 3))) =
        make_uint2(lo[i], hi[i]);
  }
}

template <int D, bool kCausal>
__global__ void __launch_bounds__(64 * kShortWaves, 1)
short_kernel(Bf16View q, Bf16View k, Bf16View v, int64_t H, int64_t S, int64_t S_pad, int smooth_k, float sl2,
             Bf16OutView o, float* __restrict__ lse) {
  using Gm = Geo<D>;
  using Dm = Dim<D>;
  constexpr int TB = Dm::kTileBytes, NT = Short<D>::kTiles, NW = kShortWaves;
  constexpr int QB = 32 * D;   // one resident query block
  // [K tiles][V tiles][query blocks]; during the prologue steps the per-wave
  // channel statistics and the exact-sum digits overlay the V tiles
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * NT * TB + Short<D>::kBlocks * QB];
  __shared__ float s_kmean[D], s_vinv[D], s_vlift[D], s_vscale[D];
  __shared__ __attribute__((aligned(16))) float s_qscale[Short<D>::kBlocks], s_kscale[Short<D>::kBlocks];
  static_assert(NW * D * (sizeof(double) + sizeof(float)) <= NT * TB, "statistics overlay");
  static_assert(kExactSlices * kDigits * D * sizeof(long long) <= NT * TB, "digit overlay");
  uint8_t* const kres = lds;
  uint8_t* const vres = lds + NT * TB;
  uint8_t* const qres = lds + 2 * NT * TB;
  double(*const fsum)[D] = reinterpret_cast<double(*)[D]>(vres);
  float(*const fmx)[D] = reinterpret_cast<float(*)[D]>(vres + NW * D * sizeof(double));
  long long(*const dig)[kDigits][D] = reinterpret_cast<long long(*)[kDigits][D]>(vres);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x, b = bh / H, h = bh % H;
  const int nt = (int)(S_pad / kKvTile), nb = 4 * nt;   // key tiles, 32-row blocks
  const int c = lane % Gm::L, g = lane / Gm::L;
  const uint16_t* qb = q.data + b * q.sb + h * q.sh + 8 * c;
  const uint16_t* kb = k.data + b * k.sb + h * k.sh + 8 * c;
  const uint16_t* vb = v.data + b * v.sb + h * v.sh + 8 * c;

  // ---- Q codes, K codes when smooth_k is off, channel statistics: piece
  // p = 3 j + t is tensor t (Q, K, V) of block j
  double ksum[8];
  float vmax[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { ksum[e] = 0.0; vmax[e] = 0.0f; }
  const int npa = 3 * nb;
  auto load_piece = [&](int p, Row16 (&r)[Gm::I]) {
    const int j = p / 3, t = p - 3 * j;
    const int64_t r0 = 32 * (int64_t)j;
    if (t == 0) {   // Q is read once: nontemporal
#pragma unroll
      for (int i = 0; i < Gm::I; ++i) {
        const int64_t row = r0 + Gm::G * i + g;
        r[i] = row < S ? load16nt(qb + row * q.ss) : Row16{{0, 0, 0, 0}};
      }
    } else if (t == 1) {
#pragma unroll
      for (int i = 0; i < Gm::I; ++i) {
        const int64_t row = r0 + Gm::G * i + g;
        r[i] = row < S ? load16(kb + row * k.ss) : Row16{{0, 0, 0, 0}};
      }
    } else {   // V in the row order of its encoding below: slot i is row 4 G (i / 4) + 4 g + i % 4
#pragma unroll
      for (int i = 0; i < Gm::I; ++i) {
        const int64_t row = r0 + 4 * Gm::G * (i >> 2) + 4 * g + (i & 3);
        r[i] = row < S ? load16(vb + row * v.ss) : Row16{{0, 0, 0, 0}};
      }
    }
  };
  // The V blocks a wave reads (pieces 3 j + 2 = w mod NW: j = j0, j0 + NW,
  // ...) stay in its registers until their codes can be formed (the first NK
  // of them; the others are read again then).
  constexpr int NV = Short<D>::kVPerWave, NK = Short<D>::kVKept;
  const int j0 = (3 * (w + NW - 2)) % NW;   // 3 is its own inverse mod 8
  static_assert(NW == 8, "the V block of a wave assumes eight waves");
  Row16 vkeep[NK][Gm::I];
  // the next piece is loaded during the current one where registers allow
  constexpr bool kAhead = D == 64;
  Row16 cur[Gm::I];
  if (kAhead && w < npa) load_piece(w, cur);
  for (int p = w; p < npa; p += NW) {
    Row16 nxt[Gm::I];
    if (kAhead && p + NW < npa) load_piece(p + NW, nxt);
    if (!kAhead) load_piece(p, cur);
    const int j = p / 3, t = p - 3 * j;
    float x[8 * Gm::I];
#pragma unroll
    for (int i = 0; i < Gm::I; ++i) unpack(cur[i], &x[i * 8]);
    if (t == 0) {
      uint32_t lo[Gm::I], hi[Gm::I];
      const float sc = quant_block_codes<D>(x, lo, hi);
      if (lane == 0) s_qscale[j] = sc;
      put_q_rows<D>(qres + j * QB, lo, hi, c, g);
    } else if (t == 1) {
      if (smooth_k) {
#pragma unroll
        for (int i = 0; i < Gm::I; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) ksum[e] = add_exact_or_nan(ksum[e], (double)x[i * 8 + e]);
      } else {
        uint32_t lo[Gm::I], hi[Gm::I];
        const float sc = quant_block_codes<D>(x, lo, hi);
        if (lane == 0) s_kscale[j] = sc;
        put_k_rows<D>(kres, j, lo, hi, c, g);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8 * Gm::I; ++i) vmax[i & 7] = fmaxf(vmax[i & 7], fabsf(x[i]));
      const int slot = (j - j0) / NW;   // uniform over the wave
#pragma unroll
      for (int sl = 0; sl < NK; ++sl)
        if (slot == sl) {
#pragma unroll
          for (int i = 0; i < Gm::I; ++i) vkeep[sl][i] = cur[i];
        }
    }
    if (kAhead) {
#pragma unroll
      for (int i = 0; i < Gm::I; ++i) cur[i] = nxt[i];
    }
  }
  // the wave's statistics, folded over the lanes of a channel, then over the
  // waves in order (every addition checked, as in the three passes)
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int m = Gm::L; m < 64; m <<= 1) {
      ksum[e] = add_exact_or_nan(ksum[e], __shfl_xor(ksum[e], m, 64));
      vmax[e] = fmaxf(vmax[e], __shfl_xor(vmax[e], m, 64));
    }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { fsum[w][8 * c + e] = ksum[e]; fmx[w][8 * c + e] = vmax[e]; }
  }
  __syncthreads();
  const int d = tid % D, js = tid / D;
  double ssum = 0.0;
  float amax = 0.0f;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    ssum = add_exact_or_nan(ssum, fsum[ww][d]);
    amax = fmaxf(amax, fmx[ww][d]);
  }
  // a NaN sum: that channel is summed exactly from K (rare; uniform branch).
  // The barrier ends every read of the statistics before the digits reuse
  // their LDS.
  const bool redo = smooth_k && ssum != ssum;
  if (__syncthreads_or(redo)) {
    if (js < kExactSlices) {
#pragma unroll
      for (int kk = 0; kk < kDigits; ++kk) dig[js][kk][d] = 0;
      if (redo) exact_sum_rows(k.data + b * k.sb + h * k.sh + d, k.ss, S, js, &dig[js][0][d], D);
    }
    __syncthreads();
    if (redo) {
      long long wd[kDigits];
#pragma unroll
      for (int kk = 0; kk < kDigits; ++kk) {
        long long t = 0;
#pragma unroll
        for (int i = 0; i < kExactSlices; ++i) t += dig[i][kk][d];
        wd[kk] = t;
      }
      ssum = digits_to_double(wd);
    }
  }
  if (tid < D) {
    s_kmean[tid] = smooth_k ? (float)(ssum / (double)S) : 0.0f;
    s_vscale[tid] = amax == 0.0f ? 0.0f : amax / 448.0f;
    const float lift = amax < kTiny ? kTinyLift : 1.0f;
    s_vinv[tid] = amax == 0.0f ? 0.0f : 448.0f / (amax * lift);
    s_vlift[tid] = lift;
  }
  __syncthreads();   // the constants are in place; the overlay is free for the V tiles

  // ---- K codes when smooth_k is on (block j by wave j mod NW), then the
  // codes of the wave's V blocks from its registers
  if (smooth_k) {
    float km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) km[e] = s_kmean[8 * c + e];
    for (int j = w; j < nb; j += NW) {
      const int64_t r0 = 32 * (int64_t)j;
      float x[8 * Gm::I];
#pragma unroll
      for (int i = 0; i < Gm::I; ++i) {
        const int64_t row = r0 + Gm::G * i + g;
        float y[8];
        if (row < S) {
          unpack(load16(kb + row * k.ss), y);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[i * 8 + e] = y[e] - km[e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[i * 8 + e] = 0.0f;   // padding rows stay zero
        }
      }
      uint32_t lo[Gm::I], hi[Gm::I];
      const float sc = quant_block_codes<D>(x, lo, hi);
      if (lane == 0) s_kscale[j] = sc;
      put_k_rows<D>(kres, j, lo, hi, c, g);
    }
  }
  {
    // V: lane (c, g) converts rows 32 (j % 4) + 4 G half + 4 g + u (u = 0..3)
    // of tile j / 4, channels 8c..8c+7, as the quantize pass does; a channel's
    // four consecutive keys go to its resident row as one dword, key chunk
    // (r / 16) at slot (r / 16) XOR ((channel / 2) % 8)
    float inv[8], lift[8];
    uint32_t keep[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      inv[e] = s_vinv[8 * c + e];
      lift[e] = s_vlift[8 * c + e];
      keep[e] = inv[e] != 0.0f ? 0xFFFFFFFFu : 0u;
    }
    bool lifted = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) lifted |= lift[e] != 1.0f;
    lifted = __builtin_amdgcn_ballot_w64(lifted) != 0;
#pragma unroll
    for (int sl = 0; sl < NV; ++sl) {
      const int j = j0 + NW * sl;
      if (j >= nb) break;
      uint8_t* vtile = vres + (j >> 2) * TB;
#pragma unroll
      for (int half = 0; half < 8 / Gm::G; ++half) {
        const int rl = 32 * (j & 3) + 4 * Gm::G * half + 4 * g;   // tile row of u = 0
        uint32_t codes[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) codes[e] = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float y[8];
          if (sl < NK) {   // (the index is clamped only so that the branch not taken stays in bounds)
            unpack(vkeep[sl < NK ? sl : 0][4 * half + u], y);   // padding rows were read as zeros
          } else {
            const int64_t row = 32 * (int64_t)j + 4 * Gm::G * half + 4 * g + u;
            if (row < S) unpack(load16(vb + row * v.ss), y);
            else {
#pragma unroll
              for (int e = 0; e < 8; ++e) y[e] = 0.0f;
            }
          }
          if (lifted) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= lift[e];
          }
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[e] * inv[e], y[e + 1] * inv[e + 1], 0, false);
            codes[e] |= (pk & 0xFFu) << (8 * u);
            codes[e + 1] |= ((pk >> 8) & 0xFFu) << (8 * u);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ch = 8 * c + e;
          *reinterpret_cast<uint32_t*>(vtile + ch * kKvTile + ((((rl >> 4) ^ ((ch >> 1) & 7)) << 4) | (rl & 15))) =
              codes[e] & keep[e];
        }
      }
    }
  }
  __syncthreads();   // every wave's codes and scales are in place

  // ---- attention, per 32-query block, over the resident tiles
  const int half = lane >> 5, col = lane & 31;
  const int prow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
  const int last_valid = (int)(S - (int64_t)(nt - 1) * kKvTile);
  const float* ks = s_kscale;
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, kBufferWord3);
  const uint32_t no_off[Dm::kCopyInstr] = {};
  for (int j = w; j < nb; j += NW) {
    const uint8_t* qrow = qres + j * QB + col * D;
    const int wt = j & 3;                          // the block's place in its 128-query tile
    const int ntw = kCausal ? (j >> 2) + 1 : nt;   // key tiles the block visits
    float qs = s_qscale[j];
    const uint32_t kexact = __builtin_amdgcn_readfirstlane(__float_as_uint(0x1p-7f / (sl2 * qs)));
    asm volatile("" : "+v"(qs));
    uint32_t kmax = 0;
    for (int i = lane; i < 4 * ntw; i += 64) kmax = max(kmax, __float_as_uint(ks[i]));
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(kmax) >= kexact, 0))
      key_loop<D, kCausal, true, true>(kres, vres, none, none, no_off, no_off, ks, qs, sl2, qrow, prow, wt, half, col,
                                       ntw, nt, last_valid, (uint32_t)S_pad, 32 * (int64_t)j, S, bh, b, h, s_vscale,
                                       o, lse);
    else
      key_loop<D, kCausal, false, true>(kres, vres, none, none, no_off, no_off, ks, qs, sl2, qrow, prow, wt, half,
                                        col, ntw, nt, last_valid, (uint32_t)S_pad, 32 * (int64_t)j, S, bh, b, h,
                                        s_vscale, o, lse);
  }
}

}  // namespace

bool short_fused_fits(int64_t S, int64_t D) {
  const int64_t nt = padded_len(S) / kKvTile;
  return nt >= 1 && nt <= (D == 64 ? Short<64>::kTiles : Short<128>::kTiles);
}

hipError_t launch_fused_short(const Bf16View& q, const Bf16View& k, const Bf16View& v, int64_t B, int64_t S,
                              int64_t H, int64_t D, int smooth_k, float sm_scale, bool causal, const Bf16OutView& o,
                              float* lse, hipStream_t stream) {
  const int64_t S_pad = padded_len(S);
  const float sl2 = sm_scale * kLog2e;
#define SAGE_LAUNCH(D_, CAUSAL_)                                                                               \
  hipLaunchKernelGGL((short_kernel<D_, CAUSAL_>), dim3((unsigned)(B * H)), dim3(64 * kShortWaves), 0, stream, q, k, \
                     v, H, S, S_pad, smooth_k, sl2, o, lse)
  if (D == 64) {
    if (causal) SAGE_LAUNCH(64, true);
    else SAGE_LAUNCH(64, false);
  } else {
    if (causal) SAGE_LAUNCH(128, true);
    else SAGE_LAUNCH(128, false);
  }
#undef SAGE_LAUNCH
  return hipGetLastError();
}

namespace {
}  // namespace

hipError_t launch_attention(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                            const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                            float sm_scale, bool causal, const Bf16OutView& o, float* lse, hipStream_t stream) {
  const int64_t S_pad = padded_len(S);
  const int64_t nqt = (S_pad + kQPerWg - 1) / kQPerWg;
  const int64_t nwg = B * H * nqt;
  const float sl2 = sm_scale * kLog2e;
#define SAGE_LAUNCH(D_, CAUSAL_)                                                                               \
  hipLaunchKernelGGL((attn_kernel<D_, CAUSAL_>), dim3((unsigned)nwg), dim3(kThreads), 0, stream, q8, q_scale, k8,   \
                     k_scale, v8t, v_scale, H, S, S_pad, nqt, nwg, sl2, o, lse)
  if (D == 64) {
    if (causal) SAGE_LAUNCH(64, true);
    else SAGE_LAUNCH(64, false);
  } else {
    if (causal) SAGE_LAUNCH(128, true);
    else SAGE_LAUNCH(128, false);
  }
#undef SAGE_LAUNCH
  return hipGetLastError();
}

}  // namespace sage
