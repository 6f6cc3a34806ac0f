// Dither draws of the matrix-core FQJL kernels (D-FQJL's Gaussian dither,
// "Fast Quantized Johnson-Lindenstrauss Transforms" page; the draw is
// dither_half in device_common.h).  A kernel that keeps the cos and sin of
// the 4096 dither angles in LDS reads them with one instruction instead of
// evaluating two transcendentals and the angle arithmetic per coordinate
// pair; and the dither is added with the amplitude folded into the radius.
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

// Add the dither of one word (coordinates 4w .. 4w + 3 of its key) of size
// amp to z[0..3]: per pair the radius is scaled by amp once, and each
// coordinate takes one fused multiply-add, z += (amp R) cos, z += (amp R) sin
// (R = sqrt(-2 ln u1) as in dither_half, up to float32 rounding).
// TAB: the angle's cos and sin from cs_tab (dither_angle values); otherwise
// evaluated inline with the same instructions, so both give the same sums.
template <bool TAB>
__device__ __forceinline__ void dither_word_add(uint64_t state, const float2 *cs_tab, float amp,
                                                float *z) {
  const uint64_t h = mix64(state);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t v = half == 0 ? (uint32_t)(h >> 32) : (uint32_t)h;
    // u1 = ((v >> 12) + 1) 2^-20.  With the table, as one fused multiply-add
    // (exact, so the same value): one instruction less per pair; the shift
    // is written out, since left to the compiler it becomes a shift of the
    // 64-bit word and the conversion a 64-bit one.  (In the row-mapped
    // kernel, at its register limit, that form spills.)
    float u1;
    if constexpr (TAB) {
      uint32_t a;
      asm("v_lshrrev_b32 %0, 12, %1" : "=v"(a) : "v"(v));
      u1 = fmaf((float)a, 0x1p-20f, 0x1p-20f);
    } else {
      u1 = (float)((v >> 12) + 1u) * 0x1p-20f;
    }
    // amp R = (amp sqrt(2 ln 2)) sqrt(-log2 u1): the first factor is the
    // same for every pair of the key (formed once), and the negation is a
    // source modifier of v_sqrt_f32, so a pair takes one multiply here
    const float ar =
        (amp * 1.1774100225154747f) * __builtin_amdgcn_sqrtf(-__builtin_amdgcn_logf(u1));
    const float2 cs = TAB ? cs_tab[v & 0xFFFu] : dither_angle(v & 0xFFFu);
    z[2 * half] = fmaf(ar, cs.x, z[2 * half]);
    z[2 * half + 1] = fmaf(ar, cs.y, z[2 * half + 1]);
  }
}

}  // namespace qjl
