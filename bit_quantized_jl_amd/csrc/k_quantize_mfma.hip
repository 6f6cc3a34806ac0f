// Dense QJL key quantization on the gfx950 matrix cores.
//
// Computes, for bfloat16 keys, Y = K S^T with v_mfma_f32_32x32x16_bf16
// (float32 accumulation; bf16 x bf16 products are exact), and fuses in
// registers: the sign test, packing of the signs into 32-bit words with a
// wavefront ballot, and the key norm ||k||.  This is the QJL abstract's
// "JL transform followed by sign-bit quantization" with a dense Gaussian S.
//
// Tiling.  A workgroup keeps the whole bf16 sketch in LDS (m*d*2 bytes: 64 KB
// at d=128, m=256) and its waves stream keys.  One wave owns 64 keys (two
// 32-row tiles); the keys are the MFMA A operand (rows), sketch coordinates
// the B operand (columns).  Each lane loads its A fragment straight from HBM:
// lane (r, h) = (lane % 32, lane / 32) holds the contiguous half h of key r
// (d/2 bf16 = d bytes), and MFMA step t contracts elements [8t, 8t+8) of both
// halves.  The contraction index is therefore a permutation of the key
// dimension; the B operand uses the same permutation, which the host bakes
// into the LDS image of S (build_mfma_b_layout), so every B fragment is one
// conflict-free ds_read_b128.
//
// Bits.  In the 32x32 accumulator, lane l holds column l % 32 of rows
// 8*(v/4) + (v%4) + 4*(l/32) in register v.  One v_cmp over register v thus
// yields 32 sign bits (one word) of key row 8*(v/4)+(v%4) in its low half and
// of that row + 4 in its high half.  v_writelane drops each word into lane
// "key" of a per-coordinate-tile register, so after all tiles lane L holds the
// m/32 words of key L and stores them contiguously (m/8 bytes per key).
#include "device_common.h"

namespace qjl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// Host: write S (bf16 bits, m x d row-major) in the B-operand order used by
// quantize_mfma_kernel: for coordinate tile ct (32 coordinates), step t and
// lane l = c + 32 h, the 8 values S[32 ct + c][h d/2 + 8 t + e], e < 8.
void build_mfma_b_layout(const uint16_t *S16, int d, int m, uint16_t *out) {
  if (d % 16 != 0) return;  // the MFMA path needs d % 16 == 0; image unused otherwise
  const int T = d / 16;
  for (int ct = 0; ct < m / 32; ++ct)
    for (int t = 0; t < T; ++t)
      for (int l = 0; l < 64; ++l) {
        const int c = l & 31, h = l >> 5;
        for (int e = 0; e < 8; ++e)
          out[(((size_t)ct * T + t) * 64 + l) * 8 + e] =
              S16[(size_t)(32 * ct + c) * d + h * (d / 2) + 8 * t + e];
      }
}

namespace {

constexpr int QM_WAVES = 4;
constexpr int QM_THREADS = 64 * QM_WAVES;
constexpr int QM_RT = 2;              // 32-key row tiles per wave
constexpr int QM_KEYS = 32 * QM_RT;   // keys per wave iteration

// v_writelane_b32 with an immediate lane.  The SGPR operand is normally the
// result of the v_cmp just before; a VALU read of an SGPR written by a VALU
// instruction needs two wait states on gfx950, which the compiler cannot see
// through inline asm, so the asm supplies them itself.
template <int LANE>
__device__ __forceinline__ uint32_t writelane(uint32_t v, uint32_t s) {
  asm("s_nop 1\n\tv_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "i"(LANE));
  return v;
}

template <int D, int M>
__global__ __launch_bounds__(QM_THREADS, 2) void quantize_mfma_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Simg, int64_t n,
    float *__restrict__ norms, uint32_t *__restrict__ bits) {
  constexpr int T = D / 16;   // MFMA k-steps per key
  constexpr int CT = M / 32;  // 32-coordinate tiles
  __shared__ uint4 sS[M * D / 8];
  const int tid = threadIdx.x;
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(Simg);
    for (int i = tid; i < M * D / 8; i += QM_THREADS) sS[i] = src[i];
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int64_t ntiles = (n + QM_KEYS - 1) / QM_KEYS;
  for (int64_t tile = (int64_t)blockIdx.x * QM_WAVES + wave; tile < ntiles;
       tile += (int64_t)gridDim.x * QM_WAVES) {
    const int64_t k0 = tile * QM_KEYS;
    bf16x8_t A[QM_RT][T];
    float nsq[QM_RT];
#pragma unroll
    for (int rt = 0; rt < QM_RT; ++rt) {
      const int64_t row = k0 + 32 * rt + r;
      const uint4 *src = reinterpret_cast<const uint4 *>(K + row * D + h * (D / 2));
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        uint4 v = row < n ? src[t] : make_uint4(0, 0, 0, 0);
        A[rt][t] = __builtin_bit_cast(bf16x8_t, v);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = __uint_as_float(w[q] << 16);
          const float hi = __uint_as_float(w[q] & 0xFFFF0000u);
          s = fmaf(lo, lo, s);
          s = fmaf(hi, hi, s);
        }
      }
      nsq[rt] = s;
    }
#pragma unroll
    for (int rt = 0; rt < QM_RT; ++rt) {
      const float tot = nsq[rt] + __shfl_xor(nsq[rt], 32);
      const int64_t row = k0 + 32 * rt + r;
      if (h == 0 && row < n) norms[row] = sqrtf(tot);
    }

    uint32_t Wd[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      floatx16_t acc[QM_RT];
#pragma unroll
      for (int rt = 0; rt < QM_RT; ++rt) acc[rt] = floatx16_t{};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8_t B = __builtin_bit_cast(bf16x8_t, sS[(ct * T + t) * 64 + lane]);
#pragma unroll
        for (int rt = 0; rt < QM_RT; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][t], B, acc[rt], 0, 0, 0);
      }
      uint32_t wv = 0;
#pragma unroll
      for (int rt = 0; rt < QM_RT; ++rt) {
#define QJL_BALLOT_V(V)                                                                 \
  {                                                                                     \
    const uint64_t msk = __builtin_amdgcn_ballot_w64(acc[rt][V] >= 0.f);                \
    constexpr int ra = 8 * ((V) / 4) + ((V) % 4);                                       \
    if (rt == 0) {                                                                      \
      wv = writelane<ra>(wv, (uint32_t)msk);                                            \
      wv = writelane<ra + 4>(wv, (uint32_t)(msk >> 32));                                \
    } else {                                                                            \
      wv = writelane<32 + ra>(wv, (uint32_t)msk);                                       \
      wv = writelane<32 + ra + 4>(wv, (uint32_t)(msk >> 32));                           \
    }                                                                                   \
  }
        QJL_BALLOT_V(0) QJL_BALLOT_V(1) QJL_BALLOT_V(2) QJL_BALLOT_V(3)
        QJL_BALLOT_V(4) QJL_BALLOT_V(5) QJL_BALLOT_V(6) QJL_BALLOT_V(7)
        QJL_BALLOT_V(8) QJL_BALLOT_V(9) QJL_BALLOT_V(10) QJL_BALLOT_V(11)
        QJL_BALLOT_V(12) QJL_BALLOT_V(13) QJL_BALLOT_V(14) QJL_BALLOT_V(15)
#undef QJL_BALLOT_V
      }
      Wd[ct] = wv;
    }
    const int64_t key = k0 + lane;
    if (key < n) {
      uint4 *dst = reinterpret_cast<uint4 *>(bits + key * CT);
#pragma unroll
      for (int q = 0; q < CT / 4; ++q)
        dst[q] = make_uint4(Wd[4 * q], Wd[4 * q + 1], Wd[4 * q + 2], Wd[4 * q + 3]);
    }
  }
}

template <int D, int M>
hipError_t launch_qm(const qjl_sketch *sk, const uint16_t *K, int64_t n, float *norms,
                     uint32_t *bits, hipStream_t st) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
  }
  const size_t lds = (size_t)M * D * 2;
  const int per_cu = lds <= 80 * 1024 ? 2 : 1;
  const int64_t ntiles = (n + QM_KEYS - 1) / QM_KEYS;
  const int64_t want = (ntiles + QM_WAVES - 1) / QM_WAVES;
  const int grid = (int)(want < (int64_t)cus * per_cu ? want : (int64_t)cus * per_cu);
  hipLaunchKernelGGL((quantize_mfma_kernel<D, M>), dim3(grid), dim3(QM_THREADS), 0, st, K,
                     sk->S16mfma, n, norms, bits);
  return hipGetLastError();
}

}  // namespace

bool quantize_mfma_supported(const qjl_sketch *sk, const void *K, int dtype,
                             const uint32_t *bits) {
  const HostSketch &h = sk->host;
  if (h.variant != QJL_VARIANT_DENSE || dtype != QJL_DTYPE_BF16 || h.rho > 0.f) return false;
  if (((uintptr_t)K & 15) != 0 || ((uintptr_t)bits & 15) != 0) return false;
  if (h.d == 128) return h.m == 128 || h.m == 256 || h.m == 512;
  if (h.d == 64) return h.m == 128 || h.m == 256 || h.m == 512;
  return false;
}

hipError_t launch_quantize_mfma(const qjl_sketch *sk, const void *Kv, int64_t n, float *norms,
                                uint32_t *bits, hipStream_t st) {
  const uint16_t *K = static_cast<const uint16_t *>(Kv);
  const int d = sk->host.d, m = sk->host.m;
  if (d == 128 && m == 128) return launch_qm<128, 128>(sk, K, n, norms, bits, st);
  if (d == 128 && m == 256) return launch_qm<128, 256>(sk, K, n, norms, bits, st);
  if (d == 128 && m == 512) return launch_qm<128, 512>(sk, K, n, norms, bits, st);
  if (d == 64 && m == 128) return launch_qm<64, 128>(sk, K, n, norms, bits, st);
  if (d == 64 && m == 256) return launch_qm<64, 256>(sk, K, n, norms, bits, st);
  if (d == 64 && m == 512) return launch_qm<64, 512>(sk, K, n, norms, bits, st);
  return hipErrorInvalidValue;
}

}  // namespace qjl
