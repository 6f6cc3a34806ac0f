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

// Dither (D-FQJL's Gaussian dither, "Fast Quantized Johnson-Lindenstrauss
// Transforms" page, Key concepts): coordinate j of key i gets s_ij a_j, with
// a_j the sketch's float32 magnitude |N(j)| (drawn once with the sketch) and
// s_ij a fair sign of the key's own: word u of key i is the SplitMix64 draw
// r(seed, 5, i ceil(m/64) + u), its high half the 32-bit sign word 2u and its
// low half word 2u + 1; bit j % 32 of sign word j / 32 set means s_ij = -1.
// Per key the m values are independent N(0, 1) over the sketch's draw, as
// the dithered estimator's factor sqrt(1 + rho^2) requires.

// SplitMix64 draw u of key key_index's signs (dkey = key(seed, 5)).
__device__ __forceinline__ uint64_t dither_draw(uint64_t dkey, uint64_t key_index, int m, int u) {
  return mix64(dkey + PHI * (key_index * (uint64_t)((m + 63) >> 6) + (uint64_t)u + 1));
}

// Sign word v (coordinates 32 v .. 32 v + 31) of key key_index.
__device__ __forceinline__ uint32_t dither_word(uint64_t dkey, uint64_t key_index, int m, int v) {
  const uint64_t h = dither_draw(dkey, key_index, m, v >> 1);
  return (v & 1) ? (uint32_t)h : (uint32_t)(h >> 32);
}

// z + amp s a for the coordinate at bit b of sign word sw (a = its
// magnitude, nonnegative, so its sign bit is clear): the sign bit of a is set
// from bit b (a shift and one v_and_or_b32), then one fused multiply-add.
// Every kernel adds the dither in this one form, so kernels that compute
// the same transformed coordinate agree bit for bit.
__device__ __forceinline__ float dither_fma(float z, float amp, uint32_t sw, int b, float a) {
  const uint32_t sa = __float_as_uint(a) | ((sw << (31 - b)) & 0x80000000u);
  return fmaf(amp, __uint_as_float(sa), z);
}

// z[0 .. n) += amp s a for coordinates 32 v + b0 + i of sign word sw
// (a: their magnitudes).
template <int N>
__device__ __forceinline__ void dither_add(float *z, float amp, uint32_t sw, int b0,
                                           const float *a) {
#pragma unroll
  for (int i = 0; i < N; ++i) z[i] = dither_fma(z[i], amp, sw, b0 + i, a[i]);
}

// z[0 .. 32 NW) += amp s a for the coordinates of sign words v0 .. v0 + NW - 1
// of key key_index (a: their magnitudes).  For NW >= 2, v0 is even and each
// draw serves two words.
template <int NW>
__device__ __forceinline__ void dither_words_add(float *z, float amp, uint64_t dkey,
                                                 uint64_t key_index, int m, int v0,
                                                 const float *a) {
  if constexpr (NW == 1) {
    dither_add<32>(z, amp, dither_word(dkey, key_index, m, v0), 0, a);
  } else {
    static_assert(NW % 2 == 0, "whole draws");
#pragma unroll
    for (int p = 0; p < NW; p += 2) {
      const uint64_t h = dither_draw(dkey, key_index, m, (v0 + p) >> 1);
      dither_add<32>(z + 32 * p, amp, (uint32_t)(h >> 32), 0, a + 32 * p);
      dither_add<32>(z + 32 * p + 32, amp, (uint32_t)h, 0, a + 32 * p + 32);
    }
  }
}

}  // namespace qjl
