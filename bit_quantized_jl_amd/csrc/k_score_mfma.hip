// Packed-bit score kernel on the gfx950 matrix cores, and score dispatch.
//
// Estimator (QJL abstract, Majid Daliri's scholarfeed page): for key t and
// query i of a group,
//     score = c * ||k_t|| * sum_j (2 b_tj - 1) Sq_ij,   c = sqrt(pi/2) sqrt(1+rho^2)/m.
// Decode reads every key's bits once per token, so this kernel is bound by
// HBM bandwidth (m/8 + 4 bytes in, 4 bytes out per key and query).  With one
// query per group, a per-bit select-and-add costs ~3 VALU instructions per
// bit, more than the chip can issue at full HBM rate; instead the sum runs on
// the matrix cores:
//
//   * Bits become the fp4 (e2m1) B operand of v_mfma_scale_f32_16x16x128_f8f6f4
//     with one VALU instruction per 8 bits.  From a 32-bit word w, the four
//     registers (w & 0x11111111) | 0x22222222, w & 0x22222222,
//     w & 0x44444444 and (w & 0x88888888) | 0x22222222 hold, in nibble n,
//     the e2m1 values 1 + b/2, b, 2b and 1 - 2b of bit 4n + s (s = register).
//   * The query is held exactly as integers: X_j = rint(Sq_j 2^F) with
//     |X_j| <= 2^23, split into five balanced base-32 digits L_0..L_4 in
//     [-16, 15].  The fp8 (e4m3) A operand row c carries f_s L_c(j), with
//     f_s = 4, 2, 1, -1 chosen so every product equals 2 b_j L_c(j) plus a
//     term independent of the bits; those constant terms and the -sum_j L_c(j)
//     of the estimator are folded into the accumulator's initial value.  All
//     products and partial sums are integers below 2^24, so each row of the
//     accumulator is exactly  R_c = sum_j (2 b_j - 1) L_c(j).
//   * The epilogue forms sum_c 32^(4-c) R_c (rows of one query sit in lane
//     groups 0 and 1, or 2 and 3), scales by c ||k|| 2^-F and stores.
//
// Operand layout (16x16x128, measured on gfx950): lane l holds row/column
// l % 16.  An fp4 operand (4 registers) holds contraction indices
// [32 g, 32 g + 32) of lane group g = l / 16 as nibbles 0..31; an fp8 operand
// (8 registers) holds [16 g, 16 g + 16) in bytes 0..15 and
// [64 + 16 g, 64 + 16 g + 16) in bytes 16..31.  Rows are limb rows (query
// pair member qq = row / 8, limb c = row % 8 < 5), columns are 16 keys.  Lane
// (key r, group g) takes words [T g, T g + T) of key r, one word per MFMA, so
// bit p of word (T g + t) is fp4 element 8 (p % 4) + p / 4 of MFMA t; the A
// operand builder maps each fp8 byte to that same contraction index.
#include "device_common.h"

namespace qjl {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int SM_THREADS = 256;
constexpr int SM_WAVES = 4;

// e4m3 bit pattern of an integer |v| <= 64 with at most 4 significant bits.
__device__ __forceinline__ uint32_t e4m3_of_int(int v) {
  if (v == 0) return 0u;
  const uint32_t s = v < 0 ? 0x80u : 0u;
  const int a = v < 0 ? -v : v;
  const int e = 31 - __clz(a);
  const int man = e >= 3 ? (a >> (e - 3)) & 7 : (a << (3 - e)) & 7;
  return s | (uint32_t)((e + 7) << 3) | (uint32_t)man;
}

// Balanced base-32 digit c (0 = most significant) of X, |X| <= 2^23.
__device__ __forceinline__ int digit_of(int X, int c) {
  int rem = X, L = 0;
#pragma unroll
  for (int k = 4; k >= 0; --k) {
    const int d = ((rem + 16) & 31) - 16;
    if (k == c) L = d;
    rem = (rem - d) >> 5;
  }
  return L;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int T, int QP>
__global__ __launch_bounds__(SM_THREADS) void score_mfma_kernel(
    const float *__restrict__ Sq, const uint32_t *__restrict__ bits,
    const float *__restrict__ norms, int m, int64_t G, int64_t nq, int64_t nk, int chunk,
    float cscale, float *__restrict__ out) {
  constexpr int NQ = 2 * QP;       // queries per pass
  constexpr int JP = T * 128;      // padded coordinate count
  __shared__ int sX[NQ][JP];
  __shared__ uint4 sA[QP][T][64][2];
  __shared__ int sF[NQ];
  __shared__ int sC[NQ][5];
  const int W = m / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int gq = lane >> 4;  // lane group 0..3
  const int64_t kbeg = (int64_t)blockIdx.x * chunk;
  const int64_t kend = (kbeg + chunk) < nk ? (kbeg + chunk) : nk;

  for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
    for (int64_t q0 = 0; q0 < nq; q0 += NQ) {
      const int nqp = (int)((nq - q0) < NQ ? (nq - q0) : NQ);
      __syncthreads();
      // ---- per query: exponent F, fixed-point values, digit sums C_c
      for (int qi = wave; qi < NQ; qi += SM_WAVES) {
        const bool qv = qi < nqp;
        const float *s = Sq + (g * nq + q0 + (qv ? qi : 0)) * (int64_t)m;
        float amax = 0.f;
        if (qv)
          for (int j = lane; j < m; j += 64) amax = fmaxf(amax, fabsf(s[j]));
        amax = wave_max(amax);
        int e2 = 0;
        (void)frexpf(amax, &e2);
        const int F = amax > 0.f ? 23 - e2 : 0;
        int C[5] = {0, 0, 0, 0, 0};
        for (int j = lane; j < JP; j += 64) {
          int X = 0;
          if (qv && j < m) X = (int)rintf(ldexpf(s[j], F));
          sX[qi][j] = X;
          const int wj = (j & 3) == 0 ? 5 : ((j & 3) == 3 ? 0 : 1);
          int rem = X;
#pragma unroll
          for (int k = 4; k >= 0; --k) {
            const int d = ((rem + 16) & 31) - 16;
            C[k] += wj * d;
            rem = (rem - d) >> 5;
          }
        }
#pragma unroll
        for (int k = 0; k < 5; ++k) C[k] = wave_sum(C[k]);
        if (lane == 0) {
          sF[qi] = F;
#pragma unroll
          for (int k = 0; k < 5; ++k) sC[qi][k] = C[k];
        }
      }
      __syncthreads();
      // ---- A operand fragments (limb rows) in MFMA order
      for (int idx = tid; idx < QP * T * 64; idx += SM_THREADS) {
        const int l = idx & 63;
        const int t = (idx >> 6) % T;
        const int qp = idx / (64 * T);
        const int row = l & 15, grp = l >> 4;
        const int qi = 2 * qp + (row >> 3), c = row & 7;
        uint32_t wd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (c < 5 && qi < nqp) {
#pragma unroll
          for (int e = 0; e < 32; ++e) {
            // fp8 element e of lane group grp is contraction index k; the fp4
            // operand holds k as element k % 32 of lane group k / 32.
            const int k = e < 16 ? 16 * grp + e : 64 + 16 * grp + (e - 16);
            const int gb = k >> 5, eb = k & 31;
            const int wi = T * gb + t;
            if (wi < W) {
              const int s = eb >> 3;
              const int j = 32 * wi + 4 * (eb & 7) + s;
              const int f = s == 0 ? 4 : (s == 1 ? 2 : (s == 2 ? 1 : -1));
              wd[e >> 2] |= e4m3_of_int(f * digit_of(sX[qi][j], c)) << (8 * (e & 3));
            }
          }
        }
        sA[qp][t][l][0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        sA[qp][t][l][1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
      }
      __syncthreads();
      v8i_t A[QP][T];
#pragma unroll
      for (int qp = 0; qp < QP; ++qp)
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint4 a0 = sA[qp][t][lane][0], a1 = sA[qp][t][lane][1];
          A[qp][t] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                           (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        }
      // per-lane epilogue constants: rows 4 gq + v
      float wgt[4];
      v4f_t cinit[QP];
      float qscale[QP];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int c = (4 * gq + v) & 7;
        wgt[v] = c < 5 ? (float)(1 << (5 * (4 - c))) : 0.f;
      }
#pragma unroll
      for (int qp = 0; qp < QP; ++qp) {
        const int qi = 2 * qp + (gq >> 1);
        const bool qv = qi < nqp;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = (4 * gq + v) & 7;
          cinit[qp][v] = (qv && c < 5) ? -(float)sC[qi][c] : 0.f;
        }
        qscale[qp] = qv ? ldexpf(cscale, -sF[qi]) : 0.f;
      }
      // ---- stream the keys: 16 per MFMA tile, tiles round-robin over waves
      const uint32_t *gbits = bits + g * nk * (int64_t)W;
      const float *gnorm = norms + g * nk;
      for (int64_t k0 = kbeg + 16 * wave; k0 < kend; k0 += 16 * SM_WAVES) {
        const int64_t key = k0 + (lane & 15);
        const bool kv = key < kend;
        uint32_t wb[T];
        const uint32_t *src = gbits + key * (int64_t)W + T * gq;
#pragma unroll
        for (int i = 0; i < T; ++i) wb[i] = (kv && T * gq + i < W) ? src[i] : 0u;
        const float nrm = kv ? gnorm[key] : 0.f;
        v4f_t acc[QP];
#pragma unroll
        for (int qp = 0; qp < QP; ++qp) acc[qp] = cinit[qp];
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint32_t w = wb[t];
          const v8i_t B = v8i_t{(int)((w & 0x11111111u) | 0x22222222u), (int)(w & 0x22222222u),
                                (int)(w & 0x44444444u), (int)((w & 0x88888888u) | 0x22222222u),
                                0, 0, 0, 0};
#pragma unroll
          for (int qp = 0; qp < QP; ++qp)
            acc[qp] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[qp][t], B, acc[qp], 0, 4,
                                                                        0, 127, 0, 127);
        }
#pragma unroll
        for (int qp = 0; qp < QP; ++qp) {
          float e = acc[qp][0] * wgt[0];
          e = fmaf(acc[qp][1], wgt[1], e);
          e = fmaf(acc[qp][2], wgt[2], e);
          e = fmaf(acc[qp][3], wgt[3], e);
          e += __shfl_xor(e, 16);
          const int qi = 2 * qp + (gq >> 1);
          if ((gq & 1) == 0 && kv && qi < nqp)
            out[(g * nq + q0 + qi) * nk + key] = (e * qscale[qp]) * nrm;
        }
      }
    }
  }
}

template <int T, int QP>
hipError_t launch_sm(const float *Sq, const uint32_t *bits, const float *norms, int m, int64_t G,
                     int64_t nq, int64_t nk, float c, float *scores, hipStream_t st) {
  int64_t chunk = 2048;
  while (chunk > 256 && G * ((nk + chunk - 1) / chunk) < 1024) chunk /= 2;
  dim3 grid((unsigned)((nk + chunk - 1) / chunk), (unsigned)(G < 65535 ? G : 65535));
  hipLaunchKernelGGL((score_mfma_kernel<T, QP>), grid, dim3(SM_THREADS), 0, st, Sq, bits, norms, m,
                     G, nq, nk, (int)chunk, c, scores);
  return hipGetLastError();
}

template <int T>
hipError_t launch_sm_t(int qp, const float *Sq, const uint32_t *bits, const float *norms, int m,
                       int64_t G, int64_t nq, int64_t nk, float c, float *scores, hipStream_t st) {
  if (qp == 1) return launch_sm<T, 1>(Sq, bits, norms, m, G, nq, nk, c, scores, st);
  if (qp == 2) return launch_sm<T, 2>(Sq, bits, norms, m, G, nq, nk, c, scores, st);
  if constexpr (T <= 4) {
    if (qp == 4) return launch_sm<T, 4>(Sq, bits, norms, m, G, nq, nk, c, scores, st);
  }
  if constexpr (T <= 2) {
    if (qp == 8) return launch_sm<T, 8>(Sq, bits, norms, m, G, nq, nk, c, scores, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_score(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                        const float *norms, int64_t G, int64_t nq, int64_t nk, float *scores,
                        hipStream_t st) {
  const int m = sk->host.m;
  if (m > 1024) return launch_score_generic(sk, Sq, bits, norms, G, nq, nk, scores, st);
  const int W = m / 32;
  const int T = (W + 3) / 4;
  const int qp_max = T <= 2 ? 8 : (T <= 4 ? 4 : 2);
  int qp = 1;
  while (qp < qp_max && 2 * qp < nq) qp *= 2;
  const float c = estimator_scale(m, sk->host.rho);
  switch (T) {
    case 1: return launch_sm_t<1>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 2: return launch_sm_t<2>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 3: return launch_sm_t<3>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 4: return launch_sm_t<4>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 5: return launch_sm_t<5>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 6: return launch_sm_t<6>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 7: return launch_sm_t<7>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 8: return launch_sm_t<8>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qjl
