// Device helpers shared by the libqjl kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "qjl_internal.h"

namespace qjl {

// A launch-shape quantity (compute units, resident workgroups of a kernel)
// cached per device: each device keeps its own value, computed on first use
// with that device current.  Concurrent first uses compute the same value,
// and the relaxed atomics make that benign.
struct PerDevice {
  static constexpr int MAX_DEVICES = 64;
  std::atomic<int> v[MAX_DEVICES];
};
template <typename F>
int per_device(PerDevice &pd, F compute) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= PerDevice::MAX_DEVICES)
    return compute();
  int x = pd.v[dev].load(std::memory_order_relaxed);
  if (x == 0) {
    x = compute();
    pd.v[dev].store(x, std::memory_order_relaxed);
  }
  return x;
}

// Workgroups of `kernel` (launched with `threads` threads and no dynamic
// LDS) that the current device holds at once: compute units times the
// occupancy the runtime reports (fallbacks: 256 units, one workgroup each).
// Callers cache it per device (PerDevice).  A failed query is cleared from
// the runtime's last-error state, which the launchers report after their
// launches.
template <typename K>
int resident_workgroups(K kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu <= 0) {
    (void)hipGetLastError();
    per_cu = 1;
  }
  return cus * per_cu;
}

// Compute units of the current device (fallback 256, the failed query
// cleared as above).
inline int device_compute_units() {
  int dev = 0, cus = 0;
  (void)hipGetDevice(&dev);
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float *p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// Dither draws (D-FQJL's Gaussian dither, "Fast Quantized Johnson-Lindenstrauss
// Transforms" page).  Key i draws one SplitMix64 word per two coordinate
// pairs, h = r(seed, 4, i m/4 + w); the high 32 bits of word w serve pair 2w,
// the low 32 bits pair 2w + 1.  From a half v: u1 = ((v >> 12) + 1) 2^-20 and
// the angle 2 pi ((v & 0xFFF) + 1/2) / 4096 (both exact in float32), and
// Box-Muller returns R cos for the even and R sin for the odd coordinate, with
// R = sqrt(-2 ln u1).  The gfx950 transcendental instructions evaluate it
// directly: v_log_f32 is log2 (R^2 = -2 ln 2 log2 u1), v_sin_f32 / v_cos_f32
// take their argument in revolutions, here (2 (v & 0xFFF) + 1) 2^-13 exactly.
// Their float32 errors move a dither value by ~1e-6 of its size, far below
// the band of coordinates whose sign is not compared bit for bit.
__device__ __forceinline__ void dither_half(uint32_t v, float &xc, float &xs) {
  const float u1 = (float)((v >> 12) + 1u) * 0x1p-20f;
  const float t = (float)(2u * (v & 0xFFFu) + 1u) * 0x1p-13f;
  const float r = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u1));
  xc = r * __builtin_amdgcn_cosf(t);
  xs = r * __builtin_amdgcn_sinf(t);
}

// The four values of one word (coordinates 4w .. 4w + 3 of its key), from the
// generator's state key + PHI (ctr + 1) (stream_draw's argument to mix64): a
// loop over consecutive words forms the state once and adds multiples of
// PHI, which the compiler would otherwise fold back into a 64-bit
// multiply-add per word.
__device__ __forceinline__ void dither_word_state(uint64_t state, float (&x)[4]) {
  const uint64_t h = mix64(state);
  dither_half((uint32_t)(h >> 32), x[0], x[1]);
  dither_half((uint32_t)h, x[2], x[3]);
}

// State of word counter ctr, opaque to the optimiser (an empty asm on its
// register pair), so that state + PHI k stays one 64-bit add per word.
__device__ __forceinline__ uint64_t dither_state(uint64_t key, uint64_t ctr) {
  uint64_t s = key + PHI * (ctr + 1);
  asm volatile("" : "+v"(s));
  return s;
}

// Coordinate j of key key_index's dither (m coordinates per key).
__device__ __forceinline__ float dither_one(uint64_t key, uint64_t key_index, int m, int j) {
  const uint64_t h = mix64(key + PHI * (key_index * (uint64_t)(m / 4) + (uint64_t)(j >> 2) + 1));
  const uint32_t v = (j & 2) ? (uint32_t)h : (uint32_t)(h >> 32);
  float c, s;
  dither_half(v, c, s);
  return (j & 1) ? s : c;
}

}  // namespace qjl
