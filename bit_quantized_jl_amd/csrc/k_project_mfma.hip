// Dense query projection Sq = q S^T for bfloat16 queries on the gfx950
// matrix cores: the query's side of the QJL abstract, projected by the same
// JL matrix as the keys and left unquantized.
//
// The quantizer's contraction without the sign, on the same operand image of
// S (read from global memory: a call projects few rows, so staging S in LDS
// would cost more than it saves).  One wave per (32 queries, 32 coordinates)
// tile; the query rows are the B operand, loaded exactly as keys are.
// bf16 x bf16 products are exact and the sums accumulate in float32 in the
// quantizer's order, so a key projected here has the signs the quantizer
// stores for it.  Tile tau of the image holds, in accumulator register
// v = 4 a + b of lane (r, h), coordinate 32 (p + h W/2) + 16 s + 4 a + b
// (tau = 2 p + s): four runs of four consecutive coordinates, written as
// 16-byte stores.
#include "device_common.h"
#include "mfma_image.h"

namespace qjl {

namespace {

template <int T>
__global__ __launch_bounds__(256) void project_mfma_kernel(const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ Simg,
                                                           int m, int64_t n,
                                                           float *__restrict__ Sq) {
  constexpr int D = 16 * T;
  const int lane = threadIdx.x & 63;
  const int tau = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int W = m / 32;
  if (tau >= W) return;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + r;
  const int64_t lrow = row < n ? row : n - 1;  // rows past n re-read row n - 1, store nothing
  const uint4 *src = reinterpret_cast<const uint4 *>(q + lrow * D);
  const uint4 *img = reinterpret_cast<const uint4 *>(Simg) + (size_t)tau * T * 64 + lane;
  bf16x8_t qa[T], sa[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    qa[t] = __builtin_bit_cast(bf16x8_t, src[qm_chunk(h, t)]);
    sa[t] = __builtin_bit_cast(bf16x8_t, img[t * 64]);
  }
  floatx16_t acc = floatx16_t{};
#pragma unroll
  for (int t = 0; t < T; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[t], qa[t], acc, 0, 0, 0);
  if (row < n) {
    const int p = tau >> 1, s = tau & 1;
    float *dst = Sq + row * (int64_t)m + 32 * (p + h * (W / 2)) + 16 * s;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4 *>(dst + 4 * a) =
          float4{acc[4 * a], acc[4 * a + 1], acc[4 * a + 2], acc[4 * a + 3]};
  }
}

template <int T>
hipError_t launch_pm(const qjl_sketch *sk, const uint16_t *q, int64_t n, float *Sq,
                     hipStream_t st) {
  const int W = sk->host.m / 32;
  const dim3 grid((unsigned)((n + 31) / 32), (unsigned)((W + 3) / 4));
  hipLaunchKernelGGL(project_mfma_kernel<T>, grid, dim3(256), 0, st, q, sk->S16mfma, sk->host.m,
                     n, Sq);
  return hipGetLastError();
}

}  // namespace


bool project_mfma_supported(const qjl_sketch *sk, const void *q, int dtype, int64_t n,
                            const float *Sq) {
  const HostSketch &h = sk->host;
  if (h.variant != QJL_VARIANT_DENSE || dtype != QJL_DTYPE_BF16) return false;
  if (h.d % 16 != 0 || h.d > 256 || h.m % 64 != 0) return false;  // the image's shapes
  if (((uintptr_t)q & 15) != 0 || ((uintptr_t)Sq & 15) != 0) return false;
  return (n + 31) / 32 <= 0x7FFFFFFF;
}

hipError_t launch_project_mfma(const qjl_sketch *sk, const void *qv, int64_t n, float *Sq,
                               hipStream_t st) {
  const uint16_t *q = static_cast<const uint16_t *>(qv);
  switch (sk->host.d / 16) {
    case 1: return launch_pm<1>(sk, q, n, Sq, st);
    case 2: return launch_pm<2>(sk, q, n, Sq, st);
    case 3: return launch_pm<3>(sk, q, n, Sq, st);
    case 4: return launch_pm<4>(sk, q, n, Sq, st);
    case 5: return launch_pm<5>(sk, q, n, Sq, st);
    case 6: return launch_pm<6>(sk, q, n, Sq, st);
    case 7: return launch_pm<7>(sk, q, n, Sq, st);
    case 8: return launch_pm<8>(sk, q, n, Sq, st);
    case 9: return launch_pm<9>(sk, q, n, Sq, st);
    case 10: return launch_pm<10>(sk, q, n, Sq, st);
    case 11: return launch_pm<11>(sk, q, n, Sq, st);
    case 12: return launch_pm<12>(sk, q, n, Sq, st);
    case 13: return launch_pm<13>(sk, q, n, Sq, st);
    case 14: return launch_pm<14>(sk, q, n, Sq, st);
    case 15: return launch_pm<15>(sk, q, n, Sq, st);
    case 16: return launch_pm<16>(sk, q, n, Sq, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qjl
