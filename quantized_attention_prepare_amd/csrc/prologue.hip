// Prologue of the quantized attention forward on gfx950: BF16 Q/K -> INT8 per
// 32-row block, BF16 V -> OCP FP8 E4M3 per channel, optional smooth_k (the
// per-channel key mean, summed in fp64, subtracted from K first). Head dims 128
// and 64 (one template; a 64-channel row is covered by 8 lanes instead of 16).
//
// Method: kernels-community issue "aiter-sage-attention" (section "The
// kernel": Q/K per 32-row block, V per channel) and the SageAttention-RDNA4
// v0.4.0 release notes ("What changed": key mean summed in fp64; 64-bit
// offsets, so there is no sequence-length ceiling).
//
// Three launches, all HBM-bound streaming passes:
//   stats    one pass over Q, K, V per 128-row chunk: quantizes Q (it needs no
//            global statistic), quantizes K too when smooth_k is off, and
//            writes per-chunk partial channel statistics (fp64 key sums,
//            fp32 V absolute maxima);
//   finalize one workgroup per head folds the partials in a fixed order into
//            k_mean, v_scale and 448/amax;
//   quant    second pass over K (smooth_k) and V in reverse chunk order, so
//            the most recently read data is re-read from the memory-side cache
//            first; V codes are transposed through LDS into channel-major rows.
// Every address is computed in 64-bit arithmetic from 64-bit strides.
// Rounding follows the method's reading exactly (IEEE float division and
// multiply, rint, hardware E4M3 conversion with round to nearest even, the
// key channel sum exact before its one rounding to double), so the codes,
// scales and key means are bit-identical to the CPU oracle's.
#include "prologue_ops.hpp"

namespace sage {
namespace {

constexpr int kThreads = 256;               // 4 waves; wave w owns 32-row block w of a chunk
constexpr int kVTileStride = 132;           // LDS row stride (bytes) of the V transpose tile


template <int D>
__global__ void __launch_bounds__(kThreads)
stats_kernel(Bf16View q, Bf16View k, Bf16View v, int64_t H, int64_t S, int64_t S_pad, int chunks_per_wg,
             int64_t nparts, int smooth_k, int8_t* __restrict__ q8, float* __restrict__ q_scale,
             int8_t* __restrict__ k8, float* __restrict__ k_scale, double* __restrict__ ksum_part,
             float* __restrict__ vmax_part) {
  using Gm = Geo<D>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bh = (int64_t)blockIdx.x / nparts, part = (int64_t)blockIdx.x % nparts;
  const int64_t b = bh / H, h = bh % H;
  const int64_t nchunks = S_pad / kChunk;
  const int c = lane % Gm::L, g = lane / Gm::L;
  const uint16_t* qb = q.data + b * q.sb + h * q.sh + 8 * c;
  const uint16_t* kb = k.data + b * k.sb + h * k.sh + 8 * c;
  const uint16_t* vb = v.data + b * v.sb + h * v.sh + 8 * c;

  double ksum[8];
  float vmax[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { ksum[e] = 0.0; vmax[e] = 0.0f; }

  for (int64_t ch = part * chunks_per_wg; ch < nchunks && ch < (part + 1) * chunks_per_wg; ++ch) {
    const int64_t r0 = ch * kChunk + 32 * wave;   // first row of this wave's block
    const int64_t blk = r0 / kQBlock;
    float x[8 * Gm::I];
    // Q: quantize the block
#pragma unroll
    for (int i = 0; i < Gm::I; ++i) {
      int64_t row = r0 + Gm::G * i + g;
      Row16 r = row < S ? load16nt(qb + row * q.ss) : Row16{{0, 0, 0, 0}};
      unpack(r, &x[i * 8]);
    }
    quant_block_store<D>(x, q8 + (bh * S_pad + r0) * D, q_scale + bh * (S_pad / kQBlock) + blk, lane);
    // K: statistics (smooth_k) or quantize right away
#pragma unroll
    for (int i = 0; i < Gm::I; ++i) {
      int64_t row = r0 + Gm::G * i + g;
      Row16 r = row < S ? load16(kb + row * k.ss) : Row16{{0, 0, 0, 0}};
      unpack(r, &x[i * 8]);
    }
    if (smooth_k) {
#pragma unroll
      for (int i = 0; i < Gm::I; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) ksum[e] = add_exact_or_nan(ksum[e], (double)x[i * 8 + e]);
    } else {
      quant_block_store<D>(x, k8 + (bh * S_pad + r0) * D, k_scale + bh * (S_pad / kQBlock) + blk, lane);
    }
    // V: channel absolute maxima
#pragma unroll
    for (int i = 0; i < Gm::I; ++i) {
      int64_t row = r0 + Gm::G * i + g;
      Row16 r = row < S ? load16(vb + row * v.ss) : Row16{{0, 0, 0, 0}};
      float y[8];
      unpack(r, y);
#pragma unroll
      for (int e = 0; e < 8; ++e) vmax[e] = fmaxf(vmax[e], fabsf(y[e]));
    }
  }

  // Fold the row groups of the wave (lanes c, c + L, c + 2L, ...), then the
  // four waves. Every key-sum addition is checked: an inexact one turns the
  // partial into NaN, and the finalize kernel then sums that channel exactly.
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int m = Gm::L; m < 64; m <<= 1) {
      ksum[e] = add_exact_or_nan(ksum[e], __shfl_xor(ksum[e], m, 64));
      vmax[e] = fmaxf(vmax[e], __shfl_xor(vmax[e], m, 64));
    }
  }
  __shared__ double s_sum[4][D];
  __shared__ float s_max[4][D];
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { s_sum[wave][8 * c + e] = ksum[e]; s_max[wave][8 * c + e] = vmax[e]; }
  }
  __syncthreads();
  if (tid < D) {
    double s = add_exact_or_nan(add_exact_or_nan(add_exact_or_nan(s_sum[0][tid], s_sum[1][tid]), s_sum[2][tid]),
                                s_sum[3][tid]);
    float m = fmaxf(fmaxf(s_max[0][tid], s_max[1][tid]), fmaxf(s_max[2][tid], s_max[3][tid]));
    ksum_part[(bh * nparts + part) * D + tid] = s;
    vmax_part[(bh * nparts + part) * D + tid] = m;
  }
}

// One workgroup per head: eight slices of threads each fold every eighth
// partial (loads kept in flight by unrolling), then the eight slice results
// are folded in slice order. The order is fixed, so the result is the same on
// every run.
constexpr int kFinalizeSlices = 8;

template <int D>
__global__ void __launch_bounds__(D * kFinalizeSlices)
finalize_kernel(Bf16View k, int64_t H, int64_t S, int64_t nparts, int smooth_k, const double* __restrict__ ksum_part,
                const float* __restrict__ vmax_part, float* __restrict__ kmean, float* __restrict__ vinv,
                float* __restrict__ vlift, float* __restrict__ v_scale, float* __restrict__ k_mean_out) {
  const int64_t bh = blockIdx.x;
  const int d = threadIdx.x % D, j = threadIdx.x / D;
  double s = 0.0;
  float a = 0.0f;
#pragma unroll 8
  for (int64_t p = j; p < nparts; p += kFinalizeSlices) {
    s = add_exact_or_nan(s, ksum_part[(bh * nparts + p) * D + d]);
    a = fmaxf(a, vmax_part[(bh * nparts + p) * D + d]);
  }
  // the fold of the partials, then (only if needed) the exact sums' digit words
  __shared__ union {
    struct {
      double sum[kFinalizeSlices][D];
      float max[kFinalizeSlices][D];
    } fold;
    long long dig[kExactSlices][kDigits][D];
  } sh;
  sh.fold.sum[j][d] = s;
  sh.fold.max[j][d] = a;
  __syncthreads();
  s = sh.fold.sum[0][d];
  a = sh.fold.max[0][d];
#pragma unroll
  for (int i = 1; i < kFinalizeSlices; ++i) {
    s = add_exact_or_nan(s, sh.fold.sum[i][d]);
    a = fmaxf(a, sh.fold.max[i][d]);
  }
  // A NaN sum means some fp64 addition on the way was inexact: that channel's
  // sum is then formed exactly from K itself (the same value the fp64 sum has
  // whenever it is exact). Rare in practice; uniform over the workgroup. The
  // barrier also ends every read of the fold before the digits reuse its LDS.
  const bool redo = smooth_k && s != s;
  if (__syncthreads_or(redo)) {
    if (j < kExactSlices) {
#pragma unroll
      for (int kk = 0; kk < kDigits; ++kk) sh.dig[j][kk][d] = 0;
      if (redo) {
        const int64_t b = bh / H, h = bh % H;
        exact_sum_rows(k.data + b * k.sb + h * k.sh + d, k.ss, S, j, &sh.dig[j][0][d], D);
      }
    }
    __syncthreads();
    if (redo) {
      long long w[kDigits];
#pragma unroll
      for (int kk = 0; kk < kDigits; ++kk) {
        long long t = 0;
#pragma unroll
        for (int i = 0; i < kExactSlices; ++i) t += sh.dig[i][kk][d];
        w[kk] = t;
      }
      s = digits_to_double(w);
    }
  }
  if (j != 0) return;
  float km = smooth_k ? (float)(s / (double)S) : 0.0f;
  kmean[bh * D + d] = km;
  if (k_mean_out) k_mean_out[bh * D + d] = km;
  v_scale[bh * D + d] = a == 0.0f ? 0.0f : a / 448.0f;
  // a channel of tiny values is lifted by 2^64 before 448/a, as an INT8 block is
  const float lift = a < kTiny ? kTinyLift : 1.0f;
  vinv[bh * D + d] = a == 0.0f ? 0.0f : 448.0f / (a * lift);
  vlift[bh * D + d] = lift;
}

template <int D>
__global__ void __launch_bounds__(kThreads)
quant_kernel(Bf16View k, Bf16View v, int64_t H, int64_t S, int64_t S_pad, int smooth_k,
             const float* __restrict__ kmean, const float* __restrict__ vinv, const float* __restrict__ vlift,
             int8_t* __restrict__ k8, float* __restrict__ k_scale, uint8_t* __restrict__ v8t) {
  using Gm = Geo<D>;
  __shared__ uint32_t tile[D * kVTileStride / 4];   // [channel][row] codes, 132-byte rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nchunks = S_pad / kChunk;
  const int64_t id = (int64_t)gridDim.x - 1 - (int64_t)blockIdx.x;   // reverse of the stats order
  const int64_t bh = id / nchunks, ch = id % nchunks;
  const int64_t b = bh / H, h = bh % H;
  const int c = lane % Gm::L, g = lane / Gm::L;

  if (smooth_k) {
    const int64_t r0 = ch * kChunk + 32 * wave;
    const uint16_t* kb = k.data + b * k.sb + h * k.sh + 8 * c;
    float km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) km[e] = kmean[bh * D + 8 * c + e];
    float x[8 * Gm::I];
#pragma unroll
    for (int i = 0; i < Gm::I; ++i) {
      int64_t row = r0 + Gm::G * i + g;
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
    quant_block_store<D>(x, k8 + (bh * S_pad + r0) * D, k_scale + bh * (S_pad / kQBlock) + r0 / kQBlock, lane);
  }

  // V: lane (c, g) of wave w converts rows 32w + 4G*half + 4g + j (j = 0..3,
  // half = 0 .. 8/G - 1) of channels 8c..8c+7, so each lane owns four
  // consecutive rows per channel and can write them to the transposed tile as
  // one dword.
  {
    const uint16_t* vb = v.data + b * v.sb + h * v.sh + 8 * c;
    float inv[8], lift[8];
    uint32_t keep[8];   // an all-zero channel (scale 0) gets codes 0, also for its -0 entries
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      inv[e] = vinv[bh * D + 8 * c + e];
      lift[e] = vlift[bh * D + 8 * c + e];
      keep[e] = inv[e] != 0.0f ? 0xFFFFFFFFu : 0u;
    }
    // channels of tiny values are lifted by 2^64 before the scaling (their
    // quotient was formed from the lifted maximum); the factor is applied only
    // when some channel of the wave needs it
    bool lifted = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) lifted |= lift[e] != 1.0f;
    lifted = __builtin_amdgcn_ballot_w64(lifted) != 0;
#pragma unroll
    for (int half = 0; half < 8 / Gm::G; ++half) {
      const int rl = 32 * wave + 4 * Gm::G * half + 4 * g;   // local row of j = 0
      uint32_t codes[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) codes[e] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int64_t row = ch * kChunk + rl + j;
        float y[8];
        if (row < S) unpack(load16(vb + row * v.ss), y);
        else {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = 0.0f;
        }
        if (lifted) {
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] *= lift[e];
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          // E4M3 with round to nearest even; |y * inv| <= 448 (1 + 2^-23) never overflows
          uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[e] * inv[e], y[e + 1] * inv[e + 1], 0, false);
          codes[e] |= (pk & 0xFFu) << (8 * j);
          codes[e + 1] |= ((pk >> 8) & 0xFFu) << (8 * j);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[((8 * c + e) * kVTileStride + rl) / 4] = codes[e] & keep[e];
    }
  }
  __syncthreads();
  // write D channel rows x 128 keys; thread t moves 16-byte pieces
  uint8_t* vdst = v8t + bh * D * S_pad + ch * kChunk;
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    const int idx = i * kThreads + tid;
    const int chn = idx >> 3, piece = idx & 7;
    const uint32_t* src = &tile[(chn * kVTileStride + piece * 16) / 4];
    uint4 val = make_uint4(src[0], src[1], src[2], src[3]);
    __builtin_nontemporal_store(v4u_t{val.x, val.y, val.z, val.w}, reinterpret_cast<v4u_t*>(vdst + (int64_t)chn * S_pad + piece * 16));
  }
}

template <int D>
hipError_t launch_prologue_d(const Bf16View& q, const Bf16View& k, const Bf16View& v, const PrologueShape& ps,
                             int smooth_k, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t,
                             float* v_scale, float* k_mean_out, const PrologueWs& ws, hipStream_t stream) {
  const int64_t BH = ps.B * ps.H;
  const int64_t nchunks = ps.S_pad / kChunk;
  hipLaunchKernelGGL(stats_kernel<D>, dim3((unsigned)(BH * ps.nparts)), dim3(kThreads), 0, stream, q, k, v, ps.H,
                     ps.S, ps.S_pad, ps.chunks_per_wg, ps.nparts, smooth_k, q8, q_scale, k8, k_scale, ws.ksum_part,
                     ws.vmax_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(finalize_kernel<D>, dim3((unsigned)BH), dim3(D * kFinalizeSlices), 0, stream, k, ps.H, ps.S,
                     ps.nparts, smooth_k, ws.ksum_part, ws.vmax_part, ws.kmean, ws.vinv, ws.vlift, v_scale,
                     k_mean_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(quant_kernel<D>, dim3((unsigned)(BH * nchunks)), dim3(kThreads), 0, stream, k, v, ps.H, ps.S,
                     ps.S_pad, smooth_k, ws.kmean, ws.vinv, ws.vlift, k8, k_scale, v8t);
  return hipGetLastError();
}

}  // namespace

PrologueShape prologue_shape(int64_t B, int64_t S, int64_t H, int64_t D) {
  PrologueShape ps{};
  ps.B = B; ps.S = S; ps.H = H; ps.D = D;
  ps.S_pad = padded_len(S);
  const int64_t nchunks = ps.S_pad / kChunk;
  const int64_t total = B * H * nchunks;
  int cpw = 1;
  while (cpw < 64 && total / (2 * cpw) >= 2048) cpw *= 2;   // keep >= ~2048 statistics workgroups
  ps.chunks_per_wg = cpw;
  ps.nparts = nchunks == 0 ? 0 : (nchunks + cpw - 1) / cpw;
  return ps;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prologue_ws_bytes(const PrologueShape& ps) {
  const size_t bh = (size_t)(ps.B * ps.H), D = (size_t)ps.D;
  return align256(bh * ps.nparts * D * sizeof(double)) + align256(bh * ps.nparts * D * sizeof(float)) +
         3 * align256(bh * D * sizeof(float));
}

PrologueWs prologue_ws_carve(void* ws, const PrologueShape& ps) {
  const size_t bh = (size_t)(ps.B * ps.H), D = (size_t)ps.D;
  char* p = static_cast<char*>(ws);
  PrologueWs w{};
  w.ksum_part = reinterpret_cast<double*>(p); p += align256(bh * ps.nparts * D * sizeof(double));
  w.vmax_part = reinterpret_cast<float*>(p); p += align256(bh * ps.nparts * D * sizeof(float));
  w.kmean = reinterpret_cast<float*>(p); p += align256(bh * D * sizeof(float));
  w.vinv = reinterpret_cast<float*>(p); p += align256(bh * D * sizeof(float));
  w.vlift = reinterpret_cast<float*>(p);
  return w;
}

hipError_t launch_prologue(const Bf16View& q, const Bf16View& k, const Bf16View& v, const PrologueShape& ps,
                           int smooth_k, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t,
                           float* v_scale, float* k_mean_out, const PrologueWs& ws, hipStream_t stream) {
  if (ps.D == 64)
    return launch_prologue_d<64>(q, k, v, ps, smooth_k, q8, q_scale, k8, k_scale, v8t, v_scale, k_mean_out, ws,
                                 stream);
  return launch_prologue_d<128>(q, k, v, ps, smooth_k, q8, q_scale, k8, k_scale, v8t, v_scale, k_mean_out, ws,
                                stream);
}

}  // namespace sage
