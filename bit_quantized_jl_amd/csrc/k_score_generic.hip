// Generic score kernel: one lane per (key, query), any m % 32 == 0.
//
// score = c * ||k|| * sum_j (2 b_j - 1) Sq_j  (the QJL abstract's asymmetric
// estimator), with c = sqrt(pi/2) sqrt(1 + rho^2) / m.  The sum runs in
// float64 so this path is accurate for any m; the fast path for m <= 1024 is
// the MFMA kernel in k_score_mfma.hip.
#include "device_common.h"

namespace qjl {

namespace {

constexpr int SG_THREADS = 256;
constexpr int SG_LDS_FLOATS = 8192;  // Sq values staged per pass (32 KB)

__global__ __launch_bounds__(SG_THREADS) void score_generic_kernel(
    const float *__restrict__ Sq, const uint32_t *__restrict__ bits,
    const float *__restrict__ norms, int m, int64_t G, int64_t nq, int64_t nk, float cscale,
    float *__restrict__ out) {
  __shared__ float sSq[SG_LDS_FLOATS];
  const int64_t t = (int64_t)blockIdx.x * SG_THREADS + threadIdx.x;
  const int W = m / 32;
  const int qpass = SG_LDS_FLOATS / m > 0 ? SG_LDS_FLOATS / m : 1;
  const bool valid = t < nk;
  for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
  const int64_t key = g * nk + (valid ? t : 0);
  const double scale = valid ? (double)cscale * (double)norms[key] : 0.0;
  const uint32_t *brow = bits + key * (int64_t)W;
  for (int64_t q0 = 0; q0 < nq; q0 += qpass) {
    const int nqp = (int)((nq - q0) < qpass ? (nq - q0) : qpass);
    const bool fits = m <= SG_LDS_FLOATS;
    __syncthreads();
    if (fits)
      for (int i = threadIdx.x; i < nqp * m; i += SG_THREADS)
        sSq[i] = Sq[(g * nq + q0) * (int64_t)m + i];
    __syncthreads();
    if (!valid) continue;
    for (int qi = 0; qi < nqp; ++qi) {
      const float *s = fits ? sSq + qi * m : Sq + (g * nq + q0 + qi) * (int64_t)m;
      double acc = 0.0;
      for (int w = 0; w < W; ++w) {
        const uint32_t word = brow[w];
        for (int b = 0; b < 32; ++b) {
          const double v = (double)s[32 * w + b];
          acc += ((word >> b) & 1u) ? v : -v;
        }
      }
      out[(g * nq + q0 + qi) * nk + t] = (float)(scale * acc);
    }
  }
  }
}

}  // namespace

hipError_t launch_score_generic(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, int64_t G, int64_t nq, int64_t nk,
                                float *scores, hipStream_t st) {
  const int m = sk->host.m;
  const float c = estimator_scale(m, sk->host.rho);
  dim3 grid((unsigned)((nk + SG_THREADS - 1) / SG_THREADS), (unsigned)(G < 65535 ? G : 65535));
  hipLaunchKernelGGL(score_generic_kernel, grid, dim3(SG_THREADS), 0, st, Sq, bits, norms, m, G,
                     nq, nk, c, scores);
  return hipGetLastError();
}

}  // namespace qjl
