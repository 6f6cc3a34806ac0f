// Shared pieces of the fused decode-attention kernels (k_attention.hip: one or
// two query pairs per pass, weighted sums on the vector ALUs;
// k_attention_mq.hip: several query pairs per pass, weighted sums on the
// matrix cores).
#pragma once

#include "score_common.h"

namespace qjl {
namespace at {

constexpr int AT_DV = 128;          // value width of the fast paths
constexpr int AT_PART = AT_DV + 4;  // floats per partial: sum, M, L, padding to 16 bytes
constexpr float LOG2E = 1.4426950408889634f;

// Maximum and sum over the 16 lanes of each row (lane i exchanges with
// i ^ 1, i ^ 2, then the mirrored lane of its half-row and of its row), the
// result in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false)));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, false));
  return v;
}

// exp2(x - m) with m = -inf (nothing seen yet) giving 0 instead of NaN.
__device__ __forceinline__ float exp2_shift(float x, float m) {
  return m == -INFINITY ? 0.f : exp2f(x - m);
}

}  // namespace at

// Workspace partials of the fused paths: [G * nq][P][AT_PART].
hipError_t launch_attn_combine(const float *ws, int64_t rows, int P, float *out, hipStream_t st);

// The multi-query partial kernel (k_attention_mq.hip): m = 128 T with T in
// {1, 2, 4}, bf16 values of width 128, three or more queries per group.
// *P_out receives the partials per row it writes into ws; when it is 1 the
// kernel wrote the normalised result to out itself and no combine is needed.
hipError_t launch_attn_mq_partials(int T, const float *Sq, const uint32_t *bits,
                                   const float *norms, const uint16_t *V, int64_t G, int64_t nq,
                                   int64_t nk, float c, float sl2, float *ws, float *out,
                                   int *P_out, hipStream_t st);
int attn_mq_partials(int T, int64_t G, int64_t nk);
bool attn_mq_supported(int T);

}  // namespace qjl
