// Cost of the dither generator's parts on the vector ALUs: each lane draws
// `pairs` consecutive dither pairs with the library's own code (one SplitMix64
// word per pair, then Box-Muller with the hardware transcendentals) and folds
// them into one value, so the work cannot be optimised away.  Modes:
//   0  word and Box-Muller (what the FQJL kernels do per coordinate pair)
//   1  the SplitMix64 word alone (its two 24-bit uniforms converted)
//   2  Box-Muller alone, on uniforms from a cheap counter sequence
// Measurement code for the benchmark, not part of the method.
#include "../device_common.h"

namespace {

template <int MODE>
__global__ __launch_bounds__(256) void dither_cost_kernel(uint64_t key, int pairs,
                                                          float *__restrict__ out) {
  const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  uint64_t st = qjl::dither_state(key, tid * (uint64_t)pairs);
  uint32_t seq = (uint32_t)tid * 2654435761u;
  float acc = 0.f;
  for (int i = 0; i < pairs; ++i) {
    if (MODE == 0) {
      float c, s;
      qjl::dither_pair_state(st, c, s);
      acc += c + s;
    } else if (MODE == 1) {
      const uint64_t h = qjl::mix64(st);
      acc += (float)((uint32_t)(h >> 40) + 1u) * 0x1p-24f +
             (float)((uint32_t)(h >> 16) & 0xFFFFFFu) * 0x1p-24f;
    } else {
      seq += 0x9E3779B9u;
      const float u1 = (float)((seq >> 8) + 1u) * 0x1p-24f;
      const float u2 = (float)((seq * 0x85EBCA6Bu) >> 8) * 0x1p-24f;
      const float r = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u1));
      acc += r * __builtin_amdgcn_cosf(u2) + r * __builtin_amdgcn_sinf(u2);
    }
    st += qjl::PHI;
  }
  out[tid] = acc;
}

}  // namespace

// grid workgroups of 256 lanes, `pairs` pairs per lane; out: device float[grid * 256].
// Returns 0, or 1 for bad arguments, 2 for a launch error.
extern "C" int qjl_probe_dither_cost(int mode, int grid, int pairs, float *out, void *stream) {
  if (!out || grid < 1 || pairs < 1 || mode < 0 || mode > 2) return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t key = qjl::stream_key(0, qjl::STREAM_DITHER);
  if (mode == 0)
    hipLaunchKernelGGL(dither_cost_kernel<0>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  else if (mode == 1)
    hipLaunchKernelGGL(dither_cost_kernel<1>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  else
    hipLaunchKernelGGL(dither_cost_kernel<2>, dim3(grid), dim3(256), 0, st, key, pairs, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
