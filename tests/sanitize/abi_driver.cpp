// Drives the C ABI's host-side validation with seeded random descriptors
// (sizes, strides, dtypes, alignments, flags, null pointers, workspace sizes)
// and the documented error cases, for a build of the library whose host code
// carries AddressSanitizer and UndefinedBehaviorSanitizer. Run without a GPU:
// every call must return a documented status without reaching a launch.
// Exit status 0 means every status was in range and every message non-empty
// for an error; a sanitizer report aborts with a non-zero status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sage.h"

namespace {

uint64_t g_state = 0x243F6A8885A308D3ull;

uint64_t next() {   // xorshift64*, test data only
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 2685821657736338717ull;
}

template <class T, size_t N>
T pick(const T (&a)[N]) { return a[next() % N]; }

alignas(256) unsigned char g_host[1 << 16];   // stands in for device memory; never dereferenced by the library

void* ptr(bool misalign) { return g_host + 256 + (misalign ? 2 : 0); }

bool status_ok(int s) { return s >= SAGE_OK && s <= SAGE_ERR_DEVICE; }

}  // namespace

int main() {
  const int64_t sizes[] = {0, 1, 2, 31, 64, 96, 128, 129, 1 << 20, (int64_t(1) << 25) - 128, int64_t(1) << 25,
                           int64_t(1) << 40, INT64_MAX, -1};
  const int64_t strides[] = {0, 1, 8, 16, 128, 256, 1 << 20, int64_t(1) << 59, INT64_MAX, 7, -8};
  int bad = 0;
  for (int it = 0; it < 20000; ++it) {
    sage_tensor t[4];
    for (auto& x : t) {
      x.data = (next() % 16 == 0) ? nullptr : ptr(next() % 8 == 0);
      x.dtype = (next() % 8 == 0) ? 2 : 1;
      for (int i = 0; i < 4; ++i) x.size[i] = pick(sizes);
      if (next() % 2) x.size[3] = (next() % 2) ? 64 : 128;
      for (int i = 0; i < 3; ++i) x.stride[i] = pick(strides);
      x.stride[3] = (next() % 8 == 0) ? 2 : 1;
    }
    if (next() % 2) t[1] = t[2] = t[3] = t[0];
    const float sm = (next() % 8 == 0) ? 0.0f : 0.1f;
    const size_t ws_bytes = (next() % 2) ? size_t(1) << 20 : (next() % 2 ? 0 : SIZE_MAX);
    void* ws = (next() % 8 == 0) ? nullptr : ptr(false);
    float* lse = (next() % 4 == 0) ? nullptr : static_cast<float*>(ptr(next() % 8 == 0));
    const int causal = int(next() % 2), want_lse = int(next() % 2), smooth = int(next() % 2);
    int s = sage_attn_fused(&t[0], &t[1], &t[2], &t[3], causal, sm, want_lse, lse, smooth, ws, ws_bytes, nullptr);
    bad |= !status_ok(s) || (s != SAGE_OK && sage_last_error()[0] == 0);
    void* outs[7];
    for (auto& o : outs) o = (next() % 16 == 0) ? nullptr : ptr(next() % 16 == 0);
    s = sage_prepare(&t[0], &t[1], &t[2], smooth, static_cast<int8_t*>(outs[0]), static_cast<float*>(outs[1]),
                     static_cast<int8_t*>(outs[2]), static_cast<float*>(outs[3]), static_cast<uint8_t*>(outs[4]),
                     static_cast<float*>(outs[5]), static_cast<float*>(outs[6]), ws, ws_bytes, nullptr);
    bad |= !status_ok(s) || (s != SAGE_OK && sage_last_error()[0] == 0);
    const int64_t B = t[3].size[0], S = t[3].size[1], H = t[3].size[2], D = t[3].size[3];
    s = sage_attn_ex(static_cast<int8_t*>(outs[0]), static_cast<float*>(outs[1]), static_cast<int8_t*>(outs[2]),
                     static_cast<float*>(outs[3]), static_cast<uint8_t*>(outs[4]), static_cast<float*>(outs[5]), B, S,
                     H, D, sm, causal, &t[3], lse, nullptr);
    bad |= !status_ok(s);
    s = sage_attn_lse(static_cast<int8_t*>(outs[0]), static_cast<float*>(outs[1]), static_cast<int8_t*>(outs[2]),
                      static_cast<float*>(outs[3]), static_cast<uint8_t*>(outs[4]), static_cast<float*>(outs[5]), B, S,
                      H, D, sm, &t[3], lse, nullptr);
    bad |= !status_ok(s);
    (void)sage_fused_workspace_bytes(B, S, H, D);
    (void)sage_prepare_workspace_bytes(B, S, H, D, smooth);
    (void)sage_padded_len(S);
    bad |= std::strncmp(sage_status_string(static_cast<sage_status>(s)), "SAGE_", 5) != 0;
  }
  // null descriptors and the fixed error order
  bad |= sage_attn_fused(nullptr, nullptr, nullptr, nullptr, 0, 0.1f, 0, nullptr, 1, nullptr, 0, nullptr) !=
         SAGE_ERR_INVALID_ARGUMENT;
  bad |= sage_attn(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 64, 2, 128, 0.1f, nullptr, nullptr) !=
         SAGE_ERR_INVALID_ARGUMENT;
  std::printf(bad ? "FAIL\n" : "ok\n");
  return bad;
}
