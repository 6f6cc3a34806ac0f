// The dither's angle from a table (D-FQJL's Gaussian dither, "Fast Quantized
// Johnson-Lindenstrauss Transforms" page; the draw is dither_half in
// device_common.h).  A kernel that keeps the cos and sin of the 4096 dither
// angles in LDS reads them with one instruction instead of evaluating two
// transcendentals and the angle arithmetic per coordinate pair.
#pragma once

#include "device_common.h"

namespace qjl {

// cos and sin of dither angle a (0 <= a < 4096), 2 pi (a + 1/2) / 4096: the
// expression and instructions of dither_half (device_common.h), so a table
// of these holds exactly the values that function computes inline.
__device__ __forceinline__ float2 dither_angle(uint32_t a) {
  const float t = (float)(2u * a + 1u) * 0x1p-13f;
  return make_float2(__builtin_amdgcn_cosf(t), __builtin_amdgcn_sinf(t));
}

// dither_half with the angle's cos and sin read from a table of
// dither_angle(0 .. 4095) in LDS: one read instead of two transcendentals
// and the angle arithmetic; the radius and products as in dither_half.
__device__ __forceinline__ void dither_half_tab(uint32_t v, const float2 *cs_tab, float &xc,
                                                float &xs) {
  const float u1 = (float)((v >> 12) + 1u) * 0x1p-20f;
  const float r = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u1));
  const float2 cs = cs_tab[v & 0xFFFu];
  xc = r * cs.x;
  xs = r * cs.y;
}

// dither_word_state with the table angle.
__device__ __forceinline__ void dither_word_state_tab(uint64_t state, const float2 *cs_tab,
                                                      float (&x)[4]) {
  const uint64_t h = mix64(state);
  dither_half_tab((uint32_t)(h >> 32), cs_tab, x[0], x[1]);
  dither_half_tab((uint32_t)h, cs_tab, x[2], x[3]);
}

}  // namespace qjl
