// Plain streaming-read kernels: the measured read-bandwidth ceiling that the
// benchmark reports beside the bandwidth-bound kernels of libqjl.  Not part
// of the method; built into its own library (libqjl_probe.so).
//
// Each lane reads 16-byte vectors and folds them into one xor, kept alive by
// a store that happens only if the xor equals a constant (never, for the
// benchmark's data), so no load is optimised away and almost nothing is
// written.  Two access patterns:
//   CHUNKED     workgroup w reads one contiguous chunk, U loads per lane in
//               flight per step;
//   grid-stride every workgroup steps over the whole buffer, U loads per lane
//               in flight, consecutive workgroups on consecutive 4 KB blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int U, bool CHUNKED>
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                   uint32_t *__restrict__ sink) {
  uint32_t acc = 0;
  const int64_t tid = threadIdx.x;
  if (CHUNKED) {
    int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    per = (per + 256 * U - 1) / (256 * U) * (256 * U);
    const int64_t beg = (int64_t)blockIdx.x * per;
    const int64_t end = beg + per < n16 ? beg + per : n16;
    for (int64_t i = beg + tid; i < end; i += 256 * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = i + (int64_t)u * 256;
        v[u] = j < end ? p[j] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  } else {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + tid; i < n16; i += stride * U) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = i + (int64_t)u * stride;
        v[u] = j < n16 ? p[j] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * 256 + tid] = acc;
}

template <int U>
hipError_t launch(bool chunked, const uint4 *p, int64_t n16, int grid, uint32_t *sink,
                  hipStream_t st) {
  if (chunked)
    hipLaunchKernelGGL((read_kernel<U, true>), dim3(grid), dim3(256), 0, st, p, n16, sink);
  else
    hipLaunchKernelGGL((read_kernel<U, false>), dim3(grid), dim3(256), 0, st, p, n16, sink);
  return hipGetLastError();
}

}  // namespace

// Read `bytes` (a multiple of 16) from the 16-byte aligned device buffer
// `buf` with `grid` workgroups of 256 lanes; `sink` is a device buffer of at
// least grid * 256 uint32 (written only in the never-taken case).
// pattern: 0 chunked, 1 grid-stride; unroll: 1, 2, 4 or 8.  Returns 0 on
// success, 1 for bad arguments, 2 for a launch error.
extern "C" int qjl_probe_read(const void *buf, int64_t bytes, int pattern, int unroll, int grid,
                              uint32_t *sink, void *stream) {
  if (!buf || !sink || bytes < 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) != 0 || grid < 1 ||
      (pattern != 0 && pattern != 1))
    return 1;
  const uint4 *p = static_cast<const uint4 *>(buf);
  const int64_t n16 = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool chunked = pattern == 0;
  hipError_t e;
  switch (unroll) {
    case 1: e = launch<1>(chunked, p, n16, grid, sink, st); break;
    case 2: e = launch<2>(chunked, p, n16, grid, sink, st); break;
    case 4: e = launch<4>(chunked, p, n16, grid, sink, st); break;
    case 8: e = launch<8>(chunked, p, n16, grid, sink, st); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}
