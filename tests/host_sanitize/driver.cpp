// Host code of libqjl under AddressSanitizer and UndefinedBehaviorSanitizer,
// on the CPU: sketch generation, the explicit FQJL product, the operand
// images, the device-image layout of qjl_make_sketch, the row map of
// qjl_quantize_keys_into, and the argument checks of every entry point.
//
// Built by tests/test_host_sanitizers.py from api.cpp, sketch_host.cpp and
// images_host.cpp with this file, which stands in for the HIP runtime
// (device memory is host memory: hipMalloc is malloc, hipMemcpy memcpy) and
// for the kernel launchers (they record their arguments and launch nothing).
// Exits 0 when every check holds; a sanitizer report aborts it.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../bit_quantized_jl_amd/csrc/qjl_internal.h"

// ---------------------------------------------------------------- HIP stand-ins
extern "C" {
hipError_t hipGetDeviceCount(int *n) { *n = 1; return hipSuccess; }
hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMalloc(void **p, size_t n) { *p = std::malloc(n ? n : 1); return *p ? hipSuccess : hipErrorOutOfMemory; }
hipError_t hipFree(void *p) { std::free(p); return hipSuccess; }
hipError_t hipMemcpy(void *dst, const void *src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
}

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

// ---------------------------------------------------------------- launcher stand-ins
namespace qjl {
static int launches = 0;
static RowMap last_map;
static int64_t last_n = -1;
hipError_t launch_quantize_generic(const qjl_sketch *, const void *, int, int64_t n, int64_t,
                                   const RowMap &map, float *, uint32_t *, hipStream_t) {
  ++launches; last_map = map; last_n = n; return hipSuccess;
}
hipError_t launch_project_dense(const qjl_sketch *, const void *, int, int64_t, float *,
                                hipStream_t) { ++launches; return hipSuccess; }
bool project_mfma_supported(const qjl_sketch *, const void *, int, int64_t, const float *) {
  return false;
}
hipError_t launch_project_mfma(const qjl_sketch *, const void *, int64_t, float *, hipStream_t) {
  ++launches; return hipSuccess;
}
bool quantize_mfma_supported(const qjl_sketch *, const void *, int, const uint32_t *) { return false; }
hipError_t launch_quantize_mfma(const qjl_sketch *, const void *, int64_t, const RowMap &, float *,
                                uint32_t *, hipStream_t) { ++launches; return hipSuccess; }
bool fqjl_mfma_supported(const qjl_sketch *, const void *, int, const uint32_t *) { return false; }
hipError_t launch_fqjl_mfma(const qjl_sketch *, const void *, int64_t, int64_t, const RowMap &,
                            float *, uint32_t *, hipStream_t) { ++launches; return hipSuccess; }
bool fqjl_project_mfma_supported(const qjl_sketch *, const void *, int, const float *) { return false; }
hipError_t launch_fqjl_project_mfma(const qjl_sketch *, const void *, int64_t, float *,
                                    hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_fqjl(const qjl_sketch *, const void *, int, int64_t n, int64_t, const RowMap &map,
                       float *, uint32_t *, float *, hipStream_t) {
  ++launches; last_map = map; last_n = n; return hipSuccess;
}
hipError_t launch_score(const qjl_sketch *, const float *, const uint32_t *, const float *, int64_t,
                        int64_t, int64_t, float *, hipStream_t) { ++launches; return hipSuccess; }
bool attention_fused_supported(const qjl_sketch *, const uint32_t *, const void *, int, int,
                               int64_t) { return false; }
size_t attention_workspace_bytes(const qjl_sketch *, int64_t G, int64_t nq, int64_t nk, int) {
  return (size_t)G * nq * nk * 4;
}
hipError_t launch_attention_fused(const qjl_sketch *, const float *, const uint32_t *,
                                  const float *, const void *, int64_t, int64_t, int64_t, float,
                                  float *, float *, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_attention_softmax(const float *, const void *, int, int, int64_t, int64_t,
                                    int64_t, float, float *, hipStream_t) {
  ++launches; return hipSuccess;
}
}  // namespace qjl

using namespace qjl;

static void sketches() {
  // Every shape class the library accepts, each variant: generation, the
  // operand images and the device layout (host memory here).
  const int dense[][2] = {{1, 32}, {16, 64}, {100, 96}, {128, 256}, {128, 512}, {256, 64}, {512, 32},
                          {64, 128}, {48, 8192}};
  for (auto &dm : dense) {
    qjl_sketch *sk = nullptr;
    CHECK(qjl_make_sketch(7, dm[0], dm[1], QJL_VARIANT_DENSE, 0.f, &sk) == QJL_OK && sk);
    std::vector<float> s32((size_t)dm[0] * dm[1]);
    std::vector<uint16_t> s16(s32.size());
    CHECK(qjl_sketch_export(sk, s32.data(), s16.data()) == QJL_OK);
    for (size_t i = 0; i < s32.size(); ++i) CHECK(f32_to_bf16_rne(s32[i]) == s16[i]);
    CHECK(qjl_destroy_sketch(sk) == QJL_OK);
  }
  const int fq[][2] = {{8, 32}, {16, 64}, {32, 96}, {64, 256}, {128, 128}, {128, 256}, {128, 512},
                       {128, 1024}, {256, 256}, {256, 512}};
  for (int variant = QJL_VARIANT_FQJL; variant <= QJL_VARIANT_PFQJL; ++variant)
    for (auto &dm : fq) {
      const float rho = variant == QJL_VARIANT_DFQJL ? 0.1f : 0.f;
      qjl_sketch *sk = nullptr;
      CHECK(qjl_make_sketch(3, dm[0], dm[1], variant, rho, &sk) == QJL_OK && sk);
      const HostSketch &h = sk->host;
      const int nb = dm[1] / dm[0];
      for (int b = 0; b < nb; ++b) {  // each P_b a permutation (the identity for D-FQJL)
        std::vector<int> seen(dm[0], 0);
        for (int c = 0; c < dm[0]; ++c) {
          const int p = h.P[(size_t)b * dm[0] + c];
          CHECK(p >= 0 && p < dm[0]);
          if (p >= 0 && p < dm[0]) ++seen[p];
          if (variant == QJL_VARIANT_DFQJL) CHECK(p == c);
        }
        for (int c = 0; c < dm[0]; ++c) CHECK(seen[c] == 1);
      }
      if (dm[0] <= 128) {  // the explicit product (export) stays bounded by ||G|| sqrt(d)
        std::vector<float> ex((size_t)dm[0] * dm[1]);
        CHECK(qjl_sketch_export(sk, ex.data(), nullptr) == QJL_OK);
        for (float v : ex) CHECK(std::isfinite(v));
      }
      CHECK(sk->Fmfma == nullptr || fqjl_mfma_image_shape(dm[0], dm[1]));
      CHECK(qjl_destroy_sketch(sk) == QJL_OK);
    }
}

static void images() {
  // The operand images written into buffers of exactly their size (in
  // qjl_make_sketch they share one allocation, where an overrun would stay
  // invisible): the dense image holds every value of S once, the FQJL image
  // only +1 and -1.
  const int dense[][2] = {{16, 64}, {64, 128}, {128, 256}, {128, 512}, {256, 64}, {48, 192}};
  for (auto &dm : dense) {
    HostSketch hs;
    hs.seed = 5; hs.d = dm[0]; hs.m = dm[1]; hs.variant = QJL_VARIANT_DENSE;
    generate_host_sketch(hs);
    const size_t md = (size_t)dm[0] * dm[1];
    std::vector<uint16_t> img(md, 0xFFFF);
    build_mfma_b_layout(hs.S16.data(), dm[0], dm[1], img.data());
    std::vector<uint16_t> a(hs.S16), b(img);
    std::sort(a.begin(), a.end());
    std::sort(b.begin(), b.end());
    CHECK(a == b);
  }
  for (int m : {128, 256, 512}) {
    HostSketch hs;
    hs.seed = 9; hs.d = 128; hs.m = m; hs.variant = QJL_VARIANT_FQJL;
    generate_host_sketch(hs);
    CHECK(fqjl_mfma_image_shape(128, m));
    std::vector<uint16_t> img((size_t)128 * m, 0);
    build_fqjl_mfma_image(hs, img.data());
    for (uint16_t v : img) CHECK(v == 0x3F80 || v == 0xBF80);
  }
}

static void validation() {
  qjl_sketch *sk = nullptr;
  CHECK(qjl_make_sketch(0, 128, 256, QJL_VARIANT_DENSE, 0.f, &sk) == QJL_OK);
  std::vector<float> buf(1 << 16);
  std::vector<uint32_t> words(1 << 16);
  float *f = buf.data();
  uint32_t *w = words.data();
  // bad arguments are rejected before any launch
  const int before = launches;
  CHECK(qjl_quantize_keys(sk, f, 1, -1, 0, f, w, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys(sk, f, 7, 4, 0, f, w, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys(sk, (char *)f + 1, 1, 4, 0, f, w, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys(sk, f, 1, 4, -3, f, w, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys_into(sk, f, 1, 2, 2, 8, 7, 0, f, w, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys_into(sk, f, 1, INT64_MAX / 4, 4, 8, 0, 0, f, w, nullptr) ==
        QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_quantize_keys_into(sk, f, 1, 1 << 20, 1 << 13, 1 << 13, 0, 0, f, w, nullptr) ==
        QJL_ERR_UNSUPPORTED);
  CHECK(qjl_project_query(sk, f, 3, 4, f, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_score(sk, f, w, f, 1, -1, 4, f, nullptr) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_score(sk, (float *)((char *)f + 2), w, f, 1, 1, 4, f, nullptr) ==
        QJL_ERR_INVALID_ARGUMENT);
  size_t need = 0;
  CHECK(qjl_decode_attention_workspace_size(sk, 2, 1, 100, 64, &need) == QJL_OK && need == 800);
  CHECK(qjl_decode_attention(sk, f, w, f, f, 0, 64, 2, 1, 100, NAN, f, need, f, nullptr) ==
        QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_decode_attention(sk, f, w, f, f, 0, 64, 2, 1, 100, 1.f, f, need - 4, f, nullptr) ==
        QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_decode_attention(sk, f, w, f, f, 0, 64, 2, 1, 0, 1.f, f, need, f, nullptr) ==
        QJL_ERR_INVALID_ARGUMENT);
  CHECK(launches == before);
  // valid calls reach their launchers with the row map the entry point formed
  CHECK(qjl_quantize_keys(sk, f, 0, 4, 0, f, w, nullptr) == QJL_OK && last_n == 4 &&
        last_map.per_group == 0);
  CHECK(qjl_quantize_keys_into(sk, f, 0, 3, 5, 40, 11, 9, f, w, nullptr) == QJL_OK &&
        last_n == 15 && last_map.per_group == 5 && last_map.stride == 40 && last_map.first == 11);
  CHECK(qjl_project_query(sk, f, 0, 4, f, nullptr) == QJL_OK);
  CHECK(qjl_score(sk, f, w, f, 1, 1, 4, f, nullptr) == QJL_OK);
  CHECK(qjl_decode_attention(sk, f, w, f, f, 0, 64, 2, 1, 100, 1.f, f, need, f, nullptr) == QJL_OK);
  CHECK(qjl_destroy_sketch(sk) == QJL_OK);
  // sketch parameters
  CHECK(qjl_make_sketch(0, 128, 250, 0, 0.f, &sk) == QJL_ERR_INVALID_ARGUMENT && sk == nullptr);
  CHECK(qjl_make_sketch(0, 512, 1024, 1, 0.f, &sk) == QJL_ERR_UNSUPPORTED && sk == nullptr);
  CHECK(qjl_make_sketch(0, 128, 256, 2, 0.f, &sk) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_make_sketch(0, 128, 256, 0, -1.f, &sk) == QJL_ERR_INVALID_ARGUMENT);
  CHECK(qjl_make_sketch(0, 128, 256, 0, INFINITY, &sk) == QJL_ERR_INVALID_ARGUMENT);
  for (int s : {-2147483647 - 1, -1, 0, 1, 2, 3, 4, 5, 99, 2147483647})
    CHECK(qjl_status_string((qjl_status)s) != nullptr);
  CHECK(std::strcmp(qjl_status_string((qjl_status)99), "QJL_ERR_UNKNOWN") == 0);
}

static void row_map() {
  // map_row against the arithmetic it stands for, over group sizes, strides
  // and offsets (32-bit division of rows below 2^32)
  const int64_t per[] = {1, 2, 3, 7, 64, 1000, 8192};
  const int64_t stride_extra[] = {0, 1, 5, 1 << 20};
  for (int64_t pg : per)
    for (int64_t se : stride_extra) {
      RowMap mp;
      mp.per_group = pg;
      mp.stride = pg + se;
      mp.first = se / 2;
      for (int64_t r : {int64_t(0), int64_t(1), pg - 1, pg, 3 * pg + 1, int64_t(4294967295)}) {
        if (r < 0) continue;
        const int64_t want = (r / pg) * mp.stride + mp.first + r % pg;
        CHECK(map_row(mp, r) == want);
      }
    }
}

int main() {
  sketches();
  images();
  validation();
  row_map();
  // bf16 rounding of special values
  CHECK(f32_to_bf16_rne(0.f) == 0x0000 && f32_to_bf16_rne(-0.f) == 0x8000);
  CHECK(f32_to_bf16_rne(1.f) == 0x3F80 && f32_to_bf16_rne(INFINITY) == 0x7F80);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer run: all checks passed\n");
  return 0;
}
