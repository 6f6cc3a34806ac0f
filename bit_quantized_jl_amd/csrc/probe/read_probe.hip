// Plain streaming-read kernels: the measured read-bandwidth ceiling that the
// benchmark reports beside the bandwidth-bound kernels of libqjl, and the
// same reads followed by plain writes (the ceiling for a kernel that reads
// and writes given byte counts).  Not part of the method; built into its own
// library (libqjl_probe.so).
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

// The reads of read_kernel, then each workgroup writes its contiguous share of
// `q` (m16 16-byte vectors in all) with non-temporal 16-byte stores, after
// its reads: the pattern of a kernel that keeps its results until its input
// is streamed (writes mixed into a read stream measured slower on this chip).
template <int U, bool CHUNKED>
__global__ __launch_bounds__(256) void read_write_kernel(const uint4 *__restrict__ p, int64_t n16,
                                                         uint4 *__restrict__ q, int64_t m16) {
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
  const int64_t per = (m16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < m16 ? beg + per : m16;
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  for (int64_t i = beg + tid; i < end; i += 256)
    __builtin_nontemporal_store(u32x4_t{acc, (uint32_t)i, acc, (uint32_t)i},
                                reinterpret_cast<u32x4_t *>(q + i));
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

namespace {
template <int U>
hipError_t launch_rw(bool chunked, const uint4 *p, int64_t n16, uint4 *q, int64_t m16, int grid,
                     hipStream_t st) {
  if (chunked)
    hipLaunchKernelGGL((read_write_kernel<U, true>), dim3(grid), dim3(256), 0, st, p, n16, q, m16);
  else
    hipLaunchKernelGGL((read_write_kernel<U, false>), dim3(grid), dim3(256), 0, st, p, n16, q,
                       m16);
  return hipGetLastError();
}
}  // namespace

// Read `bytes` from `buf`, then write `out_bytes` to `out` (both multiples of
// 16, both buffers 16-byte aligned), `grid` workgroups of 256 lanes; pattern
// and unroll as for qjl_probe_read.  Returns 0, 1 for bad arguments, 2 for a
// launch error.
extern "C" int qjl_probe_read_write(const void *buf, int64_t bytes, void *out, int64_t out_bytes,
                                    int pattern, int unroll, int grid, void *stream) {
  if (!buf || !out || bytes < 0 || bytes % 16 != 0 || out_bytes < 0 || out_bytes % 16 != 0 ||
      ((uintptr_t)buf & 15) != 0 || ((uintptr_t)out & 15) != 0 || grid < 1 ||
      (pattern != 0 && pattern != 1))
    return 1;
  const uint4 *p = static_cast<const uint4 *>(buf);
  uint4 *q = static_cast<uint4 *>(out);
  const int64_t n16 = bytes / 16, m16 = out_bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool chunked = pattern == 0;
  hipError_t e;
  switch (unroll) {
    case 1: e = launch_rw<1>(chunked, p, n16, q, m16, grid, st); break;
    case 2: e = launch_rw<2>(chunked, p, n16, q, m16, grid, st); break;
    case 4: e = launch_rw<4>(chunked, p, n16, q, m16, grid, st); break;
    case 8: e = launch_rw<8>(chunked, p, n16, q, m16, grid, st); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}
