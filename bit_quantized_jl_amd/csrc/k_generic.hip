// Generic dense-sketch kernels: any d <= 512, any m % 32 == 0, float32 or
// bfloat16 rows, optional dither.  Used for float32 keys, dithered dense
// sketches and shapes the MFMA kernel does not cover; and the dense query
// projection.
//
// y_j = sum_c x_c S[j][c] is accumulated in float32 with one fused
// multiply-add per c, in increasing c.  For quantization the sign bits of 64
// consecutive coordinates are gathered with one wavefront ballot: lanes 0-31
// give word j/32 and lanes 32-63 the next word (LSB-first, as the QJL
// abstract's sign-bit sketch packs them).
#include "device_common.h"

namespace qjl {

namespace {

constexpr int GEN_THREADS = 256;
constexpr int GEN_KEYS = 16;  // rows per block tile

template <typename T, bool DITHER, bool MAPPED>
__global__ __launch_bounds__(GEN_THREADS) void dense_generic_kernel(
    const T *__restrict__ X, const float *__restrict__ S, int d, int m, int64_t n, int64_t base,
    RowMap map, float rho, uint64_t dkey, const float *__restrict__ Dmag, float *__restrict__ norms,
    uint32_t *__restrict__ bits) {
  auto out_row = [&](int64_t r) -> int64_t { return MAPPED ? map_row(map, r) : r; };
  extern __shared__ float smem[];
  float *sX = smem;                        // [GEN_KEYS][d]
  float *sNorm = smem + GEN_KEYS * d;      // [GEN_KEYS]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int W = m / 32;
  for (int64_t tile = blockIdx.x; tile * GEN_KEYS < n; tile += gridDim.x) {
    const int64_t r0 = tile * GEN_KEYS;
    const int nr = (int)((n - r0) < GEN_KEYS ? (n - r0) : GEN_KEYS);
    for (int i = tid; i < GEN_KEYS * d; i += GEN_THREADS) {
      const int r = i / d;
      sX[i] = r < nr ? load_as_f32(X, (r0 + r) * (int64_t)d + (i - r * d)) : 0.f;
    }
    __syncthreads();
    if (tid < GEN_KEYS) {
      float s = 0.f;
      for (int c = 0; c < d; ++c) s = fmaf(sX[tid * d + c], sX[tid * d + c], s);
      const float nrm = sqrtf(s);
      sNorm[tid] = nrm;
      if (tid < nr) norms[out_row(r0 + tid)] = nrm;
    }
    __syncthreads();
    for (int jb = 0; jb < m; jb += GEN_THREADS) {
      const int j = jb + tid;
      const bool valid = j < m;
      float acc[GEN_KEYS];
#pragma unroll
      for (int r = 0; r < GEN_KEYS; ++r) acc[r] = 0.f;
      if (valid) {
        const float *Sj = S + (int64_t)j * d;
        for (int c = 0; c < d; ++c) {
          const float s = Sj[c];
#pragma unroll
          for (int r = 0; r < GEN_KEYS; ++r) acc[r] = fmaf(sX[r * d + c], s, acc[r]);
        }
      }
      const int w0 = (jb + wave * 64) / 32;  // word of lane 0 in this wave
#pragma unroll
      for (int r = 0; r < GEN_KEYS; ++r) {
        float y = acc[r];
        if (DITHER && valid)
          y = dither_fma(y, rho * sNorm[r],
                         dither_word(dkey, (uint64_t)(base + out_row(r0 + r)), m, j >> 5), j & 31,
                         Dmag[j]);
        const uint64_t msk = __ballot(valid && y >= 0.f);
        if (r < nr) {
          uint32_t *brow = bits + out_row(r0 + r) * (int64_t)W;
          if (lane == 0 && w0 < W) brow[w0] = (uint32_t)msk;
          if (lane == 32 && w0 + 1 < W) brow[w0 + 1] = (uint32_t)(msk >> 32);
        }
      }
    }
    __syncthreads();
  }
}

template <typename T, bool DITHER>
hipError_t launch_generic_t(const T *X, const float *S, int d, int m, int64_t n, int64_t base,
                            const RowMap &map, float rho, uint64_t dkey, const float *Dmag,
                            float *norms, uint32_t *bits, hipStream_t st) {
  const int64_t tiles = (n + GEN_KEYS - 1) / GEN_KEYS;
  const int grid = (int)(tiles < 8192 ? tiles : 8192);
  const size_t shmem = (size_t)(GEN_KEYS * d + GEN_KEYS) * sizeof(float);
  if (map.per_group != 0)
    hipLaunchKernelGGL((dense_generic_kernel<T, DITHER, true>), dim3(grid), dim3(GEN_THREADS),
                       shmem, st, X, S, d, m, n, base, map, rho, dkey, Dmag, norms, bits);
  else
    hipLaunchKernelGGL((dense_generic_kernel<T, DITHER, false>), dim3(grid), dim3(GEN_THREADS),
                       shmem, st, X, S, d, m, n, base, map, rho, dkey, Dmag, norms, bits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_generic(const qjl_sketch *sk, const void *K, int dtype, int64_t n,
                                   int64_t base, const RowMap &map, float *norms, uint32_t *bits,
                                   hipStream_t st) {
  const HostSketch &h = sk->host;
  const bool dith = h.rho > 0.f;
  if (dtype == QJL_DTYPE_F32) {
    const float *X = static_cast<const float *>(K);
    return dith ? launch_generic_t<float, true>(X, sk->S32, h.d, h.m, n, base, map, h.rho,
                                               sk->dither_key, sk->Dmag, norms, bits, st)
                : launch_generic_t<float, false>(X, sk->S32, h.d, h.m, n, base, map, h.rho,
                                                sk->dither_key, sk->Dmag, norms, bits, st);
  }
  const uint16_t *X = static_cast<const uint16_t *>(K);
  return dith ? launch_generic_t<uint16_t, true>(X, sk->S16f, h.d, h.m, n, base, map, h.rho,
                                                sk->dither_key, sk->Dmag, norms, bits, st)
              : launch_generic_t<uint16_t, false>(X, sk->S16f, h.d, h.m, n, base, map, h.rho,
                                                 sk->dither_key, sk->Dmag, norms, bits, st);
}

namespace {

// Query projection Sq = q S^T (the QJL abstract's unquantized JL transform of
// the query).  One block per (query, 256 coordinates); the query row sits in
// LDS and S is read transposed (S^T[c][j]) so consecutive lanes read
// consecutive addresses.  Same float32 fused multiply-add order as the
// quantizer: increasing c.
template <typename T>
__global__ __launch_bounds__(256) void project_dense_kernel(const T *__restrict__ q,
                                                            const float *__restrict__ ST, int d,
                                                            int m, int64_t n,
                                                            float *__restrict__ Sq) {
  __shared__ float sq[QJL_MAX_D];
  for (int64_t i = blockIdx.y; i < n; i += gridDim.y) {
    __syncthreads();
    for (int c = threadIdx.x; c < d; c += 256) sq[c] = load_as_f32(q, i * (int64_t)d + c);
    __syncthreads();
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j < m) {
      float acc = 0.f;
      const float *col = ST + j;
#pragma unroll 16
      for (int c = 0; c < d; ++c) acc = fmaf(sq[c], col[(int64_t)c * m], acc);
      Sq[i * (int64_t)m + j] = acc;
    }
  }
}

}  // namespace

hipError_t launch_project_dense(const qjl_sketch *sk, const void *q, int dtype, int64_t n,
                                float *Sq, hipStream_t st) {
  const HostSketch &h = sk->host;
  dim3 grid((unsigned)((h.m + 255) / 256), (unsigned)(n < 65535 ? n : 65535));
  if (dtype == QJL_DTYPE_F32)
    hipLaunchKernelGGL(project_dense_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float *>(q), sk->S32T, h.d, h.m, n, Sq);
  else
    hipLaunchKernelGGL(project_dense_kernel<uint16_t>, grid, dim3(256), 0, st,
                       static_cast<const uint16_t *>(q), sk->S16fT, h.d, h.m, n, Sq);
  return hipGetLastError();
}

}  // namespace qjl
