// C ABI of the quantized attention forward (declared in include/sage.h):
// argument validation on the host, workspace carving, launches on the
// caller's stream. Rejections follow the kernels-community issue
// "aiter-sage-attention", "What I have so far": non-BF16 inputs, unequal
// Q/K/V shapes and the wrong GPU architecture raise an error instead of
// falling back silently; head dims other than 64 and 128 likewise. Causal
// attention and the log-sum-exp output, which the issue's package rejects,
// are offered here as extensions.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sage.h"
#include "sage_internal.hpp"

namespace {

thread_local std::string g_last_error;

sage_status fail(sage_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sage_status fail(sage_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sage_status ok() {
  g_last_error.clear();
  return SAGE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b for non-negative operands; false when the product overflows int64.
bool mul_nonneg(int64_t a, int64_t b, int64_t* r) { return !__builtin_mul_overflow(a, b, r); }

// Whether the kernels can take B heads x H x S rows: every launch has at most
// B * H * S_pad / 128 workgroups, which must fit a 32-bit grid. Sizes >= 0.
bool extent_ok(int64_t B, int64_t S, int64_t H) {
  if (S > sage::kMaxSeq) return false;
  int64_t bh, tiles;
  return mul_nonneg(B, H, &bh) && mul_nonneg(bh, sage::padded_len(S) / sage::kKvTile, &tiles) &&
         tiles <= sage::kMaxTiles;
}

sage_status check_extent(int64_t B, int64_t S, int64_t H) {
  if (!extent_ok(B, S, H))
    return fail(SAGE_ERR_UNSUPPORTED, "problem too large: B=%lld S=%lld H=%lld (S <= 2^25-128, B*H*ceil(S/128) < 2^31)",
                (long long)B, (long long)S, (long long)H);
  return SAGE_OK;
}

// Step 1 checks (pointer, sizes) of a BF16 tensor argument.
sage_status check_tensor_args(const sage_tensor* t, const char* name) {
  if (!t) return fail(SAGE_ERR_INVALID_ARGUMENT, "%s: null tensor descriptor", name);
  for (int i = 0; i < 4; ++i)
    if (t->size[i] < 0) return fail(SAGE_ERR_INVALID_ARGUMENT, "%s: negative size[%d]", name, i);
  const bool empty = t->size[0] == 0 || t->size[1] == 0 || t->size[2] == 0 || t->size[3] == 0;
  int64_t n = 1;
  for (int i = 0; i < 4 && !empty; ++i)
    if (!mul_nonneg(n, t->size[i], &n))
      return fail(SAGE_ERR_INVALID_ARGUMENT, "%s: element count overflows 64 bits", name);
  if (!empty && !t->data) return fail(SAGE_ERR_INVALID_ARGUMENT, "%s: null data pointer", name);
  return SAGE_OK;
}

// Step 2 checks (what the kernels accept) of a BF16 tensor argument.
sage_status check_tensor_contract(const sage_tensor* t, const char* name, const int64_t* ref_size) {
  if (t->dtype != SAGE_BF16) return fail(SAGE_ERR_UNSUPPORTED, "%s: dtype %d is not BF16", name, t->dtype);
  if (!sage::supported_head_dim(t->size[3]))
    return fail(SAGE_ERR_UNSUPPORTED, "%s: head dim %lld is not 64 or 128", name, (long long)t->size[3]);
  if (ref_size)
    for (int i = 0; i < 4; ++i)
      if (t->size[i] != ref_size[i])
        return fail(SAGE_ERR_UNSUPPORTED, "%s: shape differs from q in dim %d (%lld vs %lld)", name, i,
                    (long long)t->size[i], (long long)ref_size[i]);
  if (t->stride[3] != 1) return fail(SAGE_ERR_UNSUPPORTED, "%s: stride[3] must be 1", name);
  if (t->size[1] > sage::kMaxSeq)
    return fail(SAGE_ERR_UNSUPPORTED, "%s: sequence length %lld exceeds 2^25 - 128", name, (long long)t->size[1]);
  for (int i = 0; i < 3; ++i)
    if (t->stride[i] < 0 || (t->stride[i] % 8) != 0)
      return fail(SAGE_ERR_UNSUPPORTED, "%s: stride[%d]=%lld is not a non-negative multiple of 8 elements", name, i,
                  (long long)t->stride[i]);
  // the last element's offset (in elements) must fit, with room, in the
  // kernels' 64-bit address arithmetic
  if (t->size[0] > 0 && t->size[1] > 0 && t->size[2] > 0 && t->size[3] > 0) {
    int64_t end = t->size[3];
    for (int i = 0; i < 3; ++i) {
      int64_t part;
      if (!mul_nonneg(t->size[i] - 1, t->stride[i], &part) || __builtin_add_overflow(end, part, &end) ||
          end > (int64_t(1) << 60))
        return fail(SAGE_ERR_UNSUPPORTED, "%s: strides reach past 2^60 elements", name);
    }
  }
  if (!aligned16(t->data)) return fail(SAGE_ERR_UNSUPPORTED, "%s: data pointer not 16-byte aligned", name);
  return SAGE_OK;
}

sage_status check_sizes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (B < 0 || S < 0 || H < 0 || D < 0) return fail(SAGE_ERR_INVALID_ARGUMENT, "negative size");
  return SAGE_OK;
}

// Step 4: the current device must be a gfx950. Looked up once per device.
sage_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(SAGE_ERR_UNSUPPORTED, "no HIP device: %s", hipGetErrorString(e));
  static std::mutex mu;
  static int known[64] = {0};   // 0 unknown, 1 gfx950, 2 other
  static char names[64][64];
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 64) return fail(SAGE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  if (!known[dev]) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(SAGE_ERR_UNSUPPORTED, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    snprintf(names[dev], sizeof names[dev], "%s", prop.gcnArchName);
    known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 && (prop.gcnArchName[6] == 0 || prop.gcnArchName[6] == ':')
                     ? 1 : 2;
  }
  if (known[dev] != 1) return fail(SAGE_ERR_UNSUPPORTED, "device %d is %s, not gfx950", dev, names[dev]);
  return SAGE_OK;
}

sage::Bf16View view(const sage_tensor* t) {
  return sage::Bf16View{static_cast<const uint16_t*>(t->data), t->stride[0], t->stride[1], t->stride[2]};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the fused call: quantized tensors, scales, then the prologue's own workspace.
struct FusedWs {
  int8_t* q8;
  int8_t* k8;
  uint8_t* v8t;
  float* q_scale;
  float* k_scale;
  float* v_scale;
  void* prologue;
};

size_t fused_bytes(int64_t B, int64_t S, int64_t H, int64_t D, FusedWs* carve, void* base) {
  const int64_t S_pad = sage::padded_len(S);
  const size_t bh = (size_t)(B * H);
  const size_t tens = align256(bh * (size_t)S_pad * (size_t)D);
  const size_t sc = align256(bh * (size_t)(S_pad / sage::kQBlock) * sizeof(float));
  const size_t vs = align256(bh * (size_t)D * sizeof(float));
  sage::PrologueShape ps = sage::prologue_shape(B, S, H, D);
  const size_t pro = sage::prologue_ws_bytes(ps);
  if (carve) {
    char* p = static_cast<char*>(base);
    carve->q8 = reinterpret_cast<int8_t*>(p); p += tens;
    carve->k8 = reinterpret_cast<int8_t*>(p); p += tens;
    carve->v8t = reinterpret_cast<uint8_t*>(p); p += tens;
    carve->q_scale = reinterpret_cast<float*>(p); p += sc;
    carve->k_scale = reinterpret_cast<float*>(p); p += sc;
    carve->v_scale = reinterpret_cast<float*>(p); p += vs;
    carve->prologue = p;
  }
  return 3 * tens + 2 * sc + vs + pro;
}

// ---- the prologue without a workspace argument
// Static scratch for the prologue's statistics (per-chunk key sums and V
// maxima, per-channel constants), for callers that cannot allocate. Each GPU
// the library runs on holds its own copy until the process ends. In host code
// the name `scratch` is only a stand-in: the device address of each GPU's copy
// comes from hipGetSymbolAddress, once per device with that device current,
// and only that address is passed to kernels.
constexpr size_t kScratchBytes = SAGE_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or null (with the error set).
void* scratch_of_current_device(sage_status* st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *st = fail(SAGE_ERR_DEVICE, "no usable current device for the static scratch (%d)", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *st = fail(SAGE_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

sage_status prepare_impl(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, int smooth_k, int8_t* q8,
                         float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t, float* v_scale, float* k_mean,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t B = q->size[0], S = q->size[1], H = q->size[2];
  sage::PrologueShape ps = sage::prologue_shape(B, S, H, q->size[3]);
  hipError_t e = sage::launch_prologue(view(q), view(k), view(v), ps, smooth_k ? 1 : 0, q8, q_scale, k8, k_scale, v8t,
                                       v_scale, k_mean, sage::prologue_ws_carve(ws, ps), stream);
  (void)ws_bytes;
  if (e != hipSuccess) return fail(SAGE_ERR_DEVICE, "prologue launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int sage_kv_tile(void) { return sage::kKvTile; }

int64_t sage_padded_len(int64_t S) { return sage::padded_len(S); }

size_t sage_prepare_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D, int smooth_k) {
  (void)smooth_k;
  if (B <= 0 || S <= 0 || H <= 0 || !sage::supported_head_dim(D) || !extent_ok(B, S, H)) return 0;
  return sage::prologue_ws_bytes(sage::prologue_shape(B, S, H, D));
}

size_t sage_fused_workspace_bytes(int64_t B, int64_t S, int64_t H, int64_t D) {
  if (B <= 0 || S <= 0 || H <= 0 || !sage::supported_head_dim(D) || !extent_ok(B, S, H)) return 0;
  return fused_bytes(B, S, H, D, nullptr, nullptr);
}

sage_status sage_prepare(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, int smooth_k, int8_t* q8,
                         float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t, float* v_scale, float* k_mean,
                         void* ws, size_t ws_bytes, void* stream) {
  sage_status s;
  if ((s = check_tensor_args(q, "q")) || (s = check_tensor_args(k, "k")) || (s = check_tensor_args(v, "v"))) return s;
  const int64_t B = q->size[0], S = q->size[1], H = q->size[2];
  const bool empty = B == 0 || S == 0 || H == 0;
  if (!empty && (!q8 || !q_scale || !k8 || !k_scale || !v8t || !v_scale))
    return fail(SAGE_ERR_INVALID_ARGUMENT, "null output pointer");
  const size_t need = sage_prepare_workspace_bytes(B, S, H, q->size[3], smooth_k);
  if (!empty && need > 0 && !ws) return fail(SAGE_ERR_INVALID_ARGUMENT, "null workspace");
  if ((s = check_tensor_contract(q, "q", nullptr)) || (s = check_tensor_contract(k, "k", q->size)) ||
      (s = check_tensor_contract(v, "v", q->size)) || (s = check_extent(B, S, H)))
    return s;
  const void* outs[] = {q8, q_scale, k8, k_scale, v8t, v_scale, k_mean, ws};
  for (const void* p : outs)
    if (p && !aligned16(p)) return fail(SAGE_ERR_UNSUPPORTED, "output or workspace pointer not 16-byte aligned");
  if (ws_bytes < need)
    return fail(SAGE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (empty) return ok();
  if ((s = check_device())) return s;
  return prepare_impl(q, k, v, smooth_k, q8, q_scale, k8, k_scale, v8t, v_scale, k_mean, ws, ws_bytes,
                      static_cast<hipStream_t>(stream));
}

sage_status sage_prepare_noalloc(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, int smooth_k,
                                 int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, uint8_t* v8t, float* v_scale,
                                 float* k_mean, void* stream) {
  sage_status s;
  if ((s = check_tensor_args(q, "q")) || (s = check_tensor_args(k, "k")) || (s = check_tensor_args(v, "v"))) return s;
  const int64_t B = q->size[0], S = q->size[1], H = q->size[2];
  const bool empty = B == 0 || S == 0 || H == 0;
  if (!empty && (!q8 || !q_scale || !k8 || !k_scale || !v8t || !v_scale))
    return fail(SAGE_ERR_INVALID_ARGUMENT, "null output pointer");
  if ((s = check_tensor_contract(q, "q", nullptr)) || (s = check_tensor_contract(k, "k", q->size)) ||
      (s = check_tensor_contract(v, "v", q->size)) || (s = check_extent(B, S, H)))
    return s;
  const void* outs[] = {q8, q_scale, k8, k_scale, v8t, v_scale, k_mean};
  for (const void* p : outs)
    if (p && !aligned16(p)) return fail(SAGE_ERR_UNSUPPORTED, "output pointer not 16-byte aligned");
  const size_t need = sage_prepare_workspace_bytes(B, S, H, q->size[3], smooth_k);
  if (need > kScratchBytes)
    return fail(SAGE_ERR_WORKSPACE_TOO_SMALL,
                "problem needs %zu bytes of scratch; the static scratch of the allocation-free prologue holds %zu",
                need, kScratchBytes);
  if (empty) return ok();
  if ((s = check_device())) return s;
  void* ws = scratch_of_current_device(&s);
  if (!ws) return s;
  return prepare_impl(q, k, v, smooth_k, q8, q_scale, k8, k_scale, v8t, v_scale, k_mean, ws, kScratchBytes,
                      static_cast<hipStream_t>(stream));
}

static sage_status attn_impl(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                             const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                             float sm_scale, bool causal, const sage_tensor* o, float* lse, bool want_lse,
                             void* stream) {
  sage_status s;
  if ((s = check_sizes(B, S, H, D))) return s;
  if ((s = check_tensor_args(o, "o"))) return s;
  const bool empty = B == 0 || S == 0 || H == 0;
  if (!empty && (!q8 || !q_scale || !k8 || !k_scale || !v8t || !v_scale))
    return fail(SAGE_ERR_INVALID_ARGUMENT, "null input pointer");
  if (want_lse && !empty && !lse) return fail(SAGE_ERR_INVALID_ARGUMENT, "null lse pointer");
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(SAGE_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  if (!sage::supported_head_dim(D)) return fail(SAGE_ERR_UNSUPPORTED, "head dim %lld is not 64 or 128", (long long)D);
  const int64_t want[4] = {B, S, H, D};
  if ((s = check_tensor_contract(o, "o", want)) || (s = check_extent(B, S, H))) return s;
  const void* ins[] = {q8, q_scale, k8, k_scale, v8t, v_scale};
  for (const void* p : ins)
    if (p && !aligned16(p)) return fail(SAGE_ERR_UNSUPPORTED, "input pointer not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(SAGE_ERR_UNSUPPORTED, "lse not 4-byte aligned");
  if (empty) return ok();
  if ((s = check_device())) return s;
  sage::Bf16OutView ov{static_cast<uint16_t*>(o->data), o->stride[0], o->stride[1], o->stride[2]};
  hipError_t e = sage::launch_attention(q8, q_scale, k8, k_scale, v8t, v_scale, B, S, H, D, sm_scale, causal, ov,
                                        want_lse ? lse : nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SAGE_ERR_DEVICE, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

sage_status sage_attn(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                      const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                      float sm_scale, const sage_tensor* o, void* stream) {
  return attn_impl(q8, q_scale, k8, k_scale, v8t, v_scale, B, S, H, D, sm_scale, false, o, nullptr, false, stream);
}

sage_status sage_attn_lse(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                          const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                          float sm_scale, const sage_tensor* o, float* lse, void* stream) {
  return attn_impl(q8, q_scale, k8, k_scale, v8t, v_scale, B, S, H, D, sm_scale, false, o, lse, true, stream);
}

sage_status sage_attn_ex(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                         const uint8_t* v8t, const float* v_scale, int64_t B, int64_t S, int64_t H, int64_t D,
                         float sm_scale, int is_causal, const sage_tensor* o, float* lse, void* stream) {
  return attn_impl(q8, q_scale, k8, k_scale, v8t, v_scale, B, S, H, D, sm_scale, is_causal != 0, o, lse,
                   lse != nullptr, stream);
}

sage_status sage_attn_fused(const sage_tensor* q, const sage_tensor* k, const sage_tensor* v, const sage_tensor* o,
                            int is_causal, float sm_scale, int return_lse, float* lse, int smooth_k, void* ws,
                            size_t ws_bytes, void* stream) {
  sage_status s;
  if ((s = check_tensor_args(q, "q")) || (s = check_tensor_args(k, "k")) || (s = check_tensor_args(v, "v")) ||
      (s = check_tensor_args(o, "o")))
    return s;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return fail(SAGE_ERR_INVALID_ARGUMENT, "sm_scale must be finite and positive");
  const int64_t B = q->size[0], S = q->size[1], H = q->size[2];
  const bool empty = B == 0 || S == 0 || H == 0;
  const size_t need = sage_fused_workspace_bytes(B, S, H, q->size[3]);
  if (!empty && !ws) return fail(SAGE_ERR_INVALID_ARGUMENT, "null workspace");
  if (return_lse && !empty && !lse) return fail(SAGE_ERR_INVALID_ARGUMENT, "return_lse set but lse is null");
  if (!return_lse && lse) return fail(SAGE_ERR_INVALID_ARGUMENT, "lse given but return_lse is 0");
  if ((s = check_tensor_contract(q, "q", nullptr)) || (s = check_tensor_contract(k, "k", q->size)) ||
      (s = check_tensor_contract(v, "v", q->size)) || (s = check_tensor_contract(o, "o", q->size)) ||
      (s = check_extent(B, S, H)))
    return s;
  if (ws && !aligned16(ws)) return fail(SAGE_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(SAGE_ERR_UNSUPPORTED, "lse not 4-byte aligned");
  if (ws_bytes < need) return fail(SAGE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (empty) return ok();
  if ((s = check_device())) return s;
  FusedWs w{};
  fused_bytes(B, S, H, q->size[3], &w, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  sage::Bf16OutView ov{static_cast<uint16_t*>(o->data), o->stride[0], o->stride[1], o->stride[2]};
  if (sage::short_fused_fits(S, q->size[3])) {
    hipError_t e = sage::launch_fused_short(view(q), view(k), view(v), B, S, H, q->size[3], smooth_k ? 1 : 0,
                                            sm_scale, is_causal != 0, ov, return_lse ? lse : nullptr, st);
    if (e != hipSuccess) return fail(SAGE_ERR_DEVICE, "fused launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  if ((s = prepare_impl(q, k, v, smooth_k, w.q8, w.q_scale, w.k8, w.k_scale, w.v8t, w.v_scale, nullptr, w.prologue,
                        ws_bytes, st)))
    return s;
  hipError_t e = sage::launch_attention(w.q8, w.q_scale, w.k8, w.k_scale, w.v8t, w.v_scale, B, S, H, q->size[3],
                                        sm_scale, is_causal != 0, ov, return_lse ? lse : nullptr, st);
  if (e != hipSuccess) return fail(SAGE_ERR_DEVICE, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* sage_status_string(sage_status s) {
  switch (s) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARGUMENT: return "SAGE_ERR_INVALID_ARGUMENT";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED";
    case SAGE_ERR_WORKSPACE_TOO_SMALL: return "SAGE_ERR_WORKSPACE_TOO_SMALL";
    case SAGE_ERR_DEVICE: return "SAGE_ERR_DEVICE";
  }
  return "SAGE_ERR_UNKNOWN";
}

const char* sage_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
