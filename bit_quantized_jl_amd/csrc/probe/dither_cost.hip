// Cost of the dither generator's parts on the vector ALUs: each lane draws
// `pairs` consecutive dither pairs with the library's own code (one SplitMix64
// word per two pairs, then Box-Muller with the hardware transcendentals) and
// folds them into one value, so the work cannot be optimised away.  Modes:
//   0  word and Box-Muller (what the FQJL kernels do per two coordinate pairs)
//   1  the SplitMix64 word alone (its four exact float32 inputs converted)
//   2  Box-Muller alone, on inputs from a cheap counter sequence
//   3  word and Box-Muller with the angle's cos and sin from an LDS table, added
//      with the amplitude folded into the radius (what the persistent
//      matrix-core FQJL kernel does with dither at m <= 256; the table is
//      built once per workgroup)
// Measurement code for the benchmark, not part of the method.
#include "../device_common.h"
#include "../dither_table.h"

namespace {

template <int MODE>
__global__ __launch_bounds__(256) void dither_cost_kernel(uint64_t key, int pairs,
                                                          float *__restrict__ out) {
  const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  __shared__ float2 sCS[MODE == 3 ? 4096 : 1];
  if (MODE == 3) {
    for (int i = threadIdx.x; i < 4096; i += 256) sCS[i] = qjl::dither_angle((uint32_t)i);
    __syncthreads();
  }
  uint64_t st = qjl::dither_state(key, tid * (uint64_t)(pairs / 2));
  uint32_t seq = (uint32_t)tid * 2654435761u;
  float acc = 0.f;
  for (int i = 0; i < pairs; i += 2) {  // two pairs per word
    if (MODE == 0) {
      float x[4];
      qjl::dither_word_state(st, x);
      acc += (x[0] + x[1]) + (x[2] + x[3]);
    } else if (MODE == 3) {
      float z[4] = {0.f, 0.f, 0.f, 0.f};
      qjl::dither_word_add<true>(st, sCS, 1.f, z);
      acc += (z[0] + z[1]) + (z[2] + z[3]);
    } else if (MODE == 1) {
      const uint64_t h = qjl::mix64(st);
      const uint32_t v[2] = {(uint32_t)(h >> 32), (uint32_t)h};
#pragma unroll
      for (int e = 0; e < 2; ++e)
        acc += (float)((v[e] >> 12) + 1u) * 0x1p-20f + (float)(2u * (v[e] & 0xFFFu) + 1u) * 0x1p-13f;
    } else {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        seq += 0x9E3779B9u;
        const float u1 = (float)((seq >> 12) + 1u) * 0x1p-20f;
        const float t = (float)(2u * ((seq * 0x85EBCA6Bu) & 0xFFFu) + 1u) * 0x1p-13f;
        const float r = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u1));
        acc += r * __builtin_amdgcn_cosf(t) + r * __builtin_amdgcn_sinf(t);
      }
    }
    st += qjl::PHI;
  }
  out[tid] = acc;
}

}  // namespace

// grid workgroups of 256 lanes, `pairs` pairs per lane (even); out: device float[grid * 256].
// Returns 0, or 1 for bad arguments, 2 for a launch error.
extern "C" int qjl_probe_dither_cost(int mode, int grid, int pairs, float *out, void *stream) {
  if (!out || grid < 1 || pairs < 2 || pairs % 2 || mode < 0 || mode > 3) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t key = qjl::stream_key(0, qjl::STREAM_DITHER);
  if (mode == 0)
    hipLaunchKernelGGL(dither_cost_kernel<0>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  else if (mode == 1)
    hipLaunchKernelGGL(dither_cost_kernel<1>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  else if (mode == 2)
    hipLaunchKernelGGL(dither_cost_kernel<2>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  else
    hipLaunchKernelGGL(dither_cost_kernel<3>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
