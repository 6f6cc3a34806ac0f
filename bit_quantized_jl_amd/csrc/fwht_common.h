// Register-resident Walsh-Hadamard butterflies and sign packing, shared by
// the FQJL kernels (vector-ALU transform and matrix-core first stage).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qjl {

// In-place unnormalised Walsh-Hadamard transform of D values in Sylvester
// (natural) order: log2(D) butterfly stages, D/2 add/subtract pairs each
// (H0 > 1: only the stages from pair distance H0 on, the earlier ones done
// by the caller).
template <int D, int H0 = 1>
__device__ __forceinline__ void fwht_reg(float (&u)[D]) {
#pragma unroll
  for (int h = H0; h < D; h <<= 1) {
#pragma unroll
    for (int i = 0; i < D; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = u[j], b = u[j + h];
        u[j] = a + b;
        u[j + h] = a - b;
      }
    }
  }
}

// Sign bits of 32 consecutive coordinates, bit t = [u[t] >= 0]: adding +0
// turns -0 into +0, then each v_alignbit_b32 shifts one sign bit in.
__device__ __forceinline__ uint32_t pack_nonneg(const float *u) {
  uint32_t word = 0;
#pragma unroll
  for (int t = 31; t >= 0; --t) word = __builtin_amdgcn_alignbit(word, __float_as_uint(u[t] + 0.0f), 31);
  return ~word;
}

}  // namespace qjl
