// Host-side checks of libkvq's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_host_sanitizers.py,
// no GPU): the set-up math (Lloyd-Max tables, seeded signs, sizes, status
// strings) and every entry point's argument validation, with the kernel
// launches replaced by stubs that record the call and touch no memory.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "kvq.h"
#include "kvq_internal.h"

// ---- stubs for the device side (no GPU in this build) ----
static int g_launches = 0;
static char g_scratch_stub[64];

extern "C" const char *hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace kvq {
hipError_t noalloc_scratch(void **ptr) {
  *ptr = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(g_scratch_stub) + 15) & ~uintptr_t(15));
  return hipSuccess;
}
hipError_t launch_append(const AppendArgs &, hipStream_t, bool *supported) {
  *supported = true;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attend(const AttendArgs &, hipStream_t, bool *supported) {
  *supported = true;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_attend_gated(const AttendArgs &, hipStream_t, bool *supported) {
  *supported = true;
  ++g_launches;
  return hipSuccess;
}
const char *attend_kernel_name(const AttendArgs &) { return "stub_kernel"; }
hipError_t launch_calibrate(const void *, int, int, int, int, int, int32_t *, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_merge(const MergeArgs &, hipStream_t, bool *supported) {
  *supported = true;
  ++g_launches;
  return hipSuccess;
}
}  // namespace kvq

// ---- checks ----
static int g_checks = 0;
#define CHECK(cond)                                                                  \
  do {                                                                               \
    ++g_checks;                                                                      \
    if (!(cond)) {                                                                   \
      std::fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, \
                   __LINE__, #cond, kvq_last_error());                               \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

template <typename T>
static T *fake(uintptr_t a) { return reinterpret_cast<T *>(a); }

static kvq_cache cache(int32_t batch, int32_t kv, int32_t d, int32_t cap, int32_t kf, int32_t vf) {
  kvq_cache c;
  std::memset(&c, 0, sizeof(c));
  c.batch = batch;
  c.kv_heads = kv;
  c.head_dim = d;
  c.capacity = cap;
  c.k_format = kf;
  c.v_format = vf;
  c.k_codes = fake<void>(0x100000);
  c.v_codes = fake<void>(0x200000);
  c.k_norms = fake<uint16_t>(0x300000);
  c.v_norms = fake<uint16_t>(0x400000);
  c.signs = fake<const int8_t>(0x500000);
  c.k_centroids = fake<const float>(0x600000);
  c.v_centroids = fake<const float>(0x700000);
  return c;
}

static void setup_math() {
  for (int bits = 1; bits <= 4; ++bits) {
    for (int d : {64, 128, 256}) {
      float c[16];
      CHECK(kvq_lloyd_max(bits, d, c) == KVQ_OK);
      const int L = 1 << bits;
      for (int i = 0; i + 1 < L; ++i) CHECK(c[i] < c[i + 1]);
      for (int i = 0; i < L; ++i) CHECK(c[i] == -c[L - 1 - i]);
      CHECK(std::fabs(c[L - 1]) * std::sqrt((float)d) < 3.f);
    }
  }
  float c[16];
  CHECK(kvq_lloyd_max(0, 128, c) == KVQ_EINVAL && std::strlen(kvq_last_error()) > 0);
  CHECK(kvq_lloyd_max(5, 128, c) == KVQ_EINVAL);
  CHECK(kvq_lloyd_max(4, 0, c) == KVQ_EINVAL);
  CHECK(kvq_lloyd_max(4, 100, c) == KVQ_OK);          // the set-up math takes any positive head_dim
  CHECK(kvq_lloyd_max(4, 128, nullptr) == KVQ_EINVAL);

  int8_t s[256];
  for (int d : {64, 128, 256}) {
    CHECK(kvq_make_signs(42, d, s) == KVQ_OK);
    for (int i = 0; i < d; ++i) CHECK(s[i] == 1 || s[i] == -1);
  }
  CHECK(kvq_make_signs(42, 0, s) == KVQ_EINVAL);
  CHECK(kvq_make_signs(42, 48, s) == KVQ_OK);
  CHECK(kvq_make_signs(42, 128, nullptr) == KVQ_EINVAL);

  CHECK(kvq_row_bytes(KVQ_LM4, 128) == 64 && kvq_row_bytes(KVQ_LM3, 256) == 96 && kvq_row_bytes(KVQ_LM2, 64) == 16);
  CHECK(kvq_row_bytes(KVQ_FP8_E4M3, 128) == 128);
  CHECK(kvq_row_bytes(7, 128) == 0 && kvq_row_bytes(KVQ_LM4, 96) == 0);
  CHECK(kvq_partials_floats(2, 4, 3, 128) == 2u * 4 * 3 * 128);
  for (int st = -3; st <= 8; ++st) CHECK(kvq_status_string((kvq_status)st) != nullptr);
}

static void append_validation() {
  kvq_cache c = cache(2, 4, 128, 1024, KVQ_LM4, KVQ_LM4);
  const void *k = fake<const void>(0x800000), *v = fake<const void>(0x900000);
  CHECK(kvq_quantize_append(nullptr, k, v, KVQ_F16, 0, 16, nullptr) == KVQ_EINVAL);
  CHECK(kvq_quantize_append(&c, nullptr, v, KVQ_F16, 0, 16, nullptr) == KVQ_EINVAL);
  CHECK(kvq_quantize_append(&c, k, v, 9, 0, 16, nullptr) == KVQ_EINVAL);
  CHECK(kvq_quantize_append(&c, k, v, KVQ_F16, 1020, 16, nullptr) == KVQ_ERANGE);
  CHECK(kvq_quantize_append(&c, k, v, KVQ_F16, -1, 16, nullptr) == KVQ_ERANGE);
  CHECK(kvq_quantize_append(&c, k, v, KVQ_F16, 0, -1, nullptr) == KVQ_EINVAL);
  CHECK(kvq_quantize_append(&c, fake<const void>(0x800001), v, KVQ_F16, 0, 16, nullptr) == KVQ_EINVAL);
  kvq_cache bad = c;
  bad.head_dim = 96;
  CHECK(kvq_quantize_append(&bad, k, v, KVQ_F16, 0, 16, nullptr) != KVQ_OK);
  bad = c;
  bad.k_norms = nullptr;
  CHECK(kvq_quantize_append(&bad, k, v, KVQ_F16, 0, 16, nullptr) != KVQ_OK);
  const int before = g_launches;
  CHECK(kvq_quantize_append(&c, k, v, KVQ_F16, 0, 16, nullptr) == KVQ_OK);
  CHECK(kvq_quantize_append(&c, k, v, KVQ_F32, 1008, 16, nullptr) == KVQ_OK);
  CHECK(g_launches == before + 2);
}

static void attention_validation() {
  kvq_cache c = cache(2, 4, 128, 1024, KVQ_LM4, KVQ_LM4);
  const void *q = fake<const void>(0xA00000);
  float *po = fake<float>(0xB00000), *pml = fake<float>(0xC00000), *out = fake<float>(0xD00000);
  float *lse = fake<float>(0xE00000);
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 6, 512, 4, 0, po, pml, nullptr) == KVQ_EINVAL);     // 6 % 4
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 8, 2048, 4, 0, po, pml, nullptr) != KVQ_OK);        // past capacity
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 8, 512, 0, 0, po, pml, nullptr) == KVQ_EINVAL);
  CHECK(kvq_decode_attention(&c, nullptr, KVQ_F16, 8, 512, 4, 0, po, pml, nullptr) == KVQ_EINVAL);
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 8, 512, 4, 0, nullptr, pml, nullptr) == KVQ_EINVAL);
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 8, 512, 4, 1, po, pml, nullptr) != KVQ_OK);          // no near tier
  int before = g_launches;
  CHECK(kvq_decode_attention(&c, q, KVQ_F16, 8, 512, 4, 0, po, pml, nullptr) == KVQ_OK);
  CHECK(kvq_merge(&c, po, pml, 8, 4, 0, out, lse, nullptr) == KVQ_OK);
  CHECK(kvq_merge(&c, po, pml, 8, 4, 0, out, nullptr, nullptr) == KVQ_OK);
  CHECK(g_launches == before + 3);
  CHECK(kvq_merge(&c, nullptr, pml, 8, 4, 0, out, lse, nullptr) == KVQ_EINVAL);
  CHECK(kvq_merge(&c, po, pml, 8, 0, 0, out, lse, nullptr) == KVQ_EINVAL);
  CHECK(kvq_merge(&c, fake<float>(0xB00004), pml, 8, 4, 0, out, lse, nullptr) == KVQ_EINVAL);

  // gated pass
  const float *gref = fake<const float>(0xF00000);
  uint32_t *bits = fake<uint32_t>(0x1000000);
  CHECK(kvq_decode_attention_gated(&c, q, KVQ_F16, 8, 512, 4, 0, nullptr, nullptr, nullptr, po, pml, nullptr) ==
        KVQ_EINVAL);
  CHECK(kvq_decode_attention_gated(&c, q, KVQ_F16, 8, 512, 4, 0, gref, gref, nullptr, po, pml, nullptr) ==
        KVQ_EINVAL);
  CHECK(kvq_decode_attention_gated(&c, q, KVQ_F16, 8, 512, 4, 0, gref, gref, bits, po, pml, nullptr) == KVQ_OK);

  // one-call decode: workspace sizes and checks
  const size_t n = kvq_decode_workspace_bytes(2, 8, 4, 0, 128);
  CHECK(n > 0 && kvq_decode_workspace_bytes(2, 8, 0, 0, 128) == 0 && kvq_decode_workspace_bytes(2, 8, 4, 0, 96) == 0);
  void *ws = fake<void>(0x2000000);
  CHECK(kvq_decode(&c, q, KVQ_F16, 8, 512, 4, 0, ws, n - 1, out, lse, nullptr) == KVQ_EINVAL);
  CHECK(kvq_decode(&c, q, KVQ_F16, 8, 512, 4, 0, nullptr, n, out, lse, nullptr) == KVQ_EINVAL);
  CHECK(kvq_decode(&c, q, KVQ_F16, 8, 512, 4, 0, fake<void>(0x2000008), n, out, lse, nullptr) == KVQ_EINVAL);
  before = g_launches;
  CHECK(kvq_decode(&c, q, KVQ_F16, 8, 512, 4, 0, ws, n, out, lse, nullptr) == KVQ_OK);
  CHECK(kvq_decode_noalloc(&c, q, KVQ_F16, 8, 512, 4, 0, out, lse, nullptr) == KVQ_OK);
  CHECK(g_launches == before + 4);
  kvq_cache big = cache(64, 64, 128, 1024, KVQ_LM4, KVQ_LM4);
  CHECK(kvq_decode_noalloc(&big, q, KVQ_F16, 64, 512, 64, 0, out, lse, nullptr) == KVQ_ERANGE);

  // kernel name: valid and invalid descriptions
  CHECK(kvq_decode_attention_kernel(&c, 8, 4, 0) != nullptr);
  CHECK(kvq_decode_attention_kernel(&c, 6, 4, 0) == nullptr);
  CHECK(kvq_decode_attention_kernel(&c, 8, 0, 0) == nullptr);
  CHECK(kvq_decode_attention_kernel(nullptr, 8, 4, 0) == nullptr);

  // outlier calibration
  int32_t *idx = fake<int32_t>(0x3000000);
  const void *keys = fake<const void>(0x4000000);
  CHECK(kvq_calibrate_outliers(&c, keys, KVQ_F16, 0, idx, nullptr) == KVQ_EINVAL);
  CHECK(kvq_calibrate_outliers(&c, nullptr, KVQ_F16, 16, idx, nullptr) == KVQ_EINVAL);
  CHECK(kvq_calibrate_outliers(&c, keys, KVQ_F16, 16, idx, nullptr) == KVQ_OK);
}

int main() {
  setup_math();
  append_validation();
  attention_validation();
  std::printf("host checks passed: %d checks, %d stub launches\n", g_checks, g_launches);
  return 0;
}
