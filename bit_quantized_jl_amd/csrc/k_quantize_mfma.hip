// Dense QJL key quantization on the gfx950 matrix cores.
//
// Computes, for bfloat16 keys, Y = K S^T with v_mfma_f32_32x32x16_bf16
// (float32 accumulation; bf16 x bf16 products are exact), and fuses in
// registers: the sign test, packing of the signs into 32-bit words with a
// wavefront ballot, and the key norm ||k||.  This is the QJL abstract's
// "JL transform followed by sign-bit quantization" with a dense Gaussian S.
//
// Tiling.  A workgroup keeps the whole bf16 sketch in LDS (m*d*2 bytes: 64 KB
// at d=128, m=256) and its waves stream keys.  S is the MFMA A operand (rows
// are sketch coordinates), keys the B operand (columns): one wave owns 64 keys
// (two 32-key column tiles).  Each lane loads its key fragment straight from
// HBM: lane (c, h) = (lane % 32, lane / 32) holds the contiguous half h of key
// c (d/2 bf16 = d bytes), and MFMA step t contracts elements [8t, 8t+8) of
// both halves.  The contraction index is therefore a permutation of the key
// dimension; the S fragments use the same permutation, which the host bakes
// into the LDS image of S (build_mfma_b_layout), so every S fragment is one
// conflict-free ds_read_b128.
//
// Bits.  In the 32x32 accumulator, lane l holds column (key) l % 32 and, in
// register v, row 8 (v/4) + 4 (l/32) + (v%4).  The host orders the rows of S
// so that, over the two accumulators of a tile pair (p, s = 1 then s = 0),
// lane half h sees the 32 coordinates of output word p + h W/2 of its key,
// register v of pass s holding coordinate 16 s + v.  Each lane then shifts
// the 32 sign bits into one word with v_alignbit_b32 (one instruction per
// bit, no cross-lane traffic): bit = 1 <=> the sign bit is 0 <=> y >= 0.  A
// key of norm 0 (all products zero) is written as all ones, so a zero of
// either sign counts as non-negative.  Lane (c, h) ends up with words
// [h W/2, (h+1) W/2) of key c and stores them contiguously.
#include "device_common.h"

namespace qjl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// Host: write S (bf16 bits, m x d row-major) in the operand order used by
// quantize_mfma_kernel.  Tile tau = 2 p + s (p < W/2 word pairs, s < 2),
// row r = 8 a + 4 h + b of the tile is coordinate 32 (p + h W/2) + 16 s + 4 a + b;
// for tile tau, step t and lane l = r + 32 hh the 8 values
// S[row][hh d/2 + 8 t + e], e < 8, are contiguous.
void build_mfma_b_layout(const uint16_t *S16, int d, int m, uint16_t *out) {
  if (d % 16 != 0 || m % 64 != 0) return;  // the MFMA path's shapes; image unused otherwise
  const int T = d / 16, W = m / 32;
  for (int tau = 0; tau < m / 32; ++tau) {
    const int p = tau >> 1, s = tau & 1;
    for (int t = 0; t < T; ++t)
      for (int l = 0; l < 64; ++l) {
        const int r = l & 31, hh = l >> 5;
        const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
        const int j = 32 * (p + h * (W / 2)) + 16 * s + 4 * a + b;
        for (int e = 0; e < 8; ++e)
          out[(((size_t)tau * T + t) * 64 + l) * 8 + e] =
              S16[(size_t)j * d + hh * (d / 2) + 8 * t + e];
      }
  }
}

namespace {

// Launch shape (compile-time; the defaults are the measured best on MI355X).
#ifndef QJL_QM_WAVES
#define QJL_QM_WAVES 4      // waves per workgroup (all share one LDS copy of S)
#endif
#ifndef QJL_QM_RT
#define QJL_QM_RT 2         // 32-key column tiles per wave (S fragments reused RT times)
#endif
#ifndef QJL_QM_PREFETCH
#define QJL_QM_PREFETCH 0   // load the next key tile while computing the current one
#endif
#ifndef QJL_QM_MINWAVES
#define QJL_QM_MINWAVES 2   // waves per SIMD the register allocation must allow
#endif
constexpr int QM_WAVES = QJL_QM_WAVES;
constexpr int QM_THREADS = 64 * QM_WAVES;
constexpr int QM_RT = QJL_QM_RT;
constexpr int QM_KEYS = 32 * QM_RT;   // keys per wave iteration

template <int T>
struct KeyTile {
  bf16x8_t a[QM_RT][T];
};

// Load the A fragments of the 64 keys starting at k0.  Rows past n re-read
// row n-1 (their results are never stored): the loads stay unconditional, so
// the compiler can count them and wait only for the tile it needs.
template <int D>
__device__ __forceinline__ void load_tile(KeyTile<D / 16> &kt, const uint16_t *__restrict__ K,
                                          int64_t k0, int64_t n, int r, int h) {
  constexpr int T = D / 16;
#pragma unroll
  for (int rt = 0; rt < QM_RT; ++rt) {
    int64_t row = k0 + 32 * rt + r;
    row = row < n ? row : n - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(K + row * D + h * (D / 2));
#pragma unroll
    for (int t = 0; t < T; ++t) kt.a[rt][t] = __builtin_bit_cast(bf16x8_t, src[t]);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Norms, projection, sign packing and stores for one 64-key tile.
template <int D, int M>
__device__ __forceinline__ void process_tile(const KeyTile<D / 16> &kt, const uint4 *sS,
                                             int64_t k0, int64_t n, int lane, int r, int h,
                                             float *__restrict__ norms,
                                             uint32_t *__restrict__ bits) {
  constexpr int T = D / 16;
  constexpr int W = M / 32;
  // Keep the LDS reads of S inside the tile loop: hoisting all m*d/512 B
  // fragments into registers would not fit and would spill.
  asm volatile("" ::: "memory");
  bool zero[QM_RT];
#pragma unroll
  for (int rt = 0; rt < QM_RT; ++rt) {
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint4 v = __builtin_bit_cast(uint4, kt.a[rt][t]);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x2_t x = __builtin_bit_cast(bf16x2_t, w[q]);
        s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
      }
    }
    const float tot = s + __shfl_xor(s, 32);
    zero[rt] = !(tot > 0.f);
    const int64_t row = k0 + 32 * rt + r;
    if (h == 0 && row < n) norms[row] = sqrtf(tot);
  }
  uint32_t Wd[QM_RT][W / 2];
#pragma unroll
  for (int p = 0; p < W / 2; ++p) {
    uint32_t x[QM_RT] = {};
#pragma unroll
    for (int s = 1; s >= 0; --s) {
      const int tau = 2 * p + s;
      asm volatile("" ::: "memory");  // bound the S fragments held in registers to one pass
      floatx16_t acc[QM_RT];
#pragma unroll
      for (int rt = 0; rt < QM_RT; ++rt) acc[rt] = floatx16_t{};
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, sS[(tau * T + t) * 64 + lane]);
#pragma unroll
        for (int rt = 0; rt < QM_RT; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, kt.a[rt][t], acc[rt], 0, 0, 0);
      }
#pragma unroll
      for (int rt = 0; rt < QM_RT; ++rt)
#pragma unroll
        for (int v = 15; v >= 0; --v)
          x[rt] = __builtin_amdgcn_alignbit(x[rt], __float_as_uint(acc[rt][v]), 31);
    }
#pragma unroll
    for (int rt = 0; rt < QM_RT; ++rt) Wd[rt][p] = zero[rt] ? 0xFFFFFFFFu : ~x[rt];
  }
#pragma unroll
  for (int rt = 0; rt < QM_RT; ++rt) {
    const int64_t key = k0 + 32 * rt + r;
    if (key < n) {
      if constexpr ((W / 2) % 4 == 0) {
        uint4 *dst = reinterpret_cast<uint4 *>(bits + key * W + h * (W / 2));
#pragma unroll
        for (int q = 0; q < W / 8; ++q)
          dst[q] = make_uint4(Wd[rt][4 * q], Wd[rt][4 * q + 1], Wd[rt][4 * q + 2],
                              Wd[rt][4 * q + 3]);
      } else {
        uint2 *dst = reinterpret_cast<uint2 *>(bits + key * W + h * (W / 2));
#pragma unroll
        for (int q = 0; q < W / 4; ++q) dst[q] = make_uint2(Wd[rt][2 * q], Wd[rt][2 * q + 1]);
      }
    }
  }
}

// Persistent kernel: each wave walks key tiles with a stride of all waves in
// the grid.  With prefetch, tile i+1 is loaded into a second register buffer
// while tile i is computed, so HBM latency overlaps the MFMA and packing work.
template <int D, int M>
__global__ __launch_bounds__(QM_THREADS, QJL_QM_MINWAVES) void quantize_mfma_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Simg, int64_t n,
    float *__restrict__ norms, uint32_t *__restrict__ bits) {
  static_assert(M % 128 == 0, "each lane stores whole 8-byte groups of words");
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
  const int64_t stride = (int64_t)gridDim.x * QM_WAVES;
  int64_t tile = (int64_t)blockIdx.x * QM_WAVES + wave;
#if QJL_QM_PREFETCH
  KeyTile<D / 16> ka, kb;
  if (tile < ntiles) load_tile<D>(ka, K, tile * QM_KEYS, n, r, h);
  while (tile < ntiles) {
    const int64_t t1 = tile + stride;
    if (t1 < ntiles) load_tile<D>(kb, K, t1 * QM_KEYS, n, r, h);
    process_tile<D, M>(ka, sS, tile * QM_KEYS, n, lane, r, h, norms, bits);
    if (t1 >= ntiles) break;
    const int64_t t2 = t1 + stride;
    if (t2 < ntiles) load_tile<D>(ka, K, t2 * QM_KEYS, n, r, h);
    process_tile<D, M>(kb, sS, t1 * QM_KEYS, n, lane, r, h, norms, bits);
    tile = t2;
  }
#else
  for (; tile < ntiles; tile += stride) {
    KeyTile<D / 16> kt;
    load_tile<D>(kt, K, tile * QM_KEYS, n, r, h);
    process_tile<D, M>(kt, sS, tile * QM_KEYS, n, lane, r, h, norms, bits);
  }
#endif
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
  int per_cu = (int)((160 * 1024) / lds);                          // LDS limit
  const int by_waves = (4 * QJL_QM_MINWAVES) / QM_WAVES;          // register limit
  per_cu = per_cu < by_waves ? per_cu : by_waves;
  per_cu = per_cu < 1 ? 1 : per_cu;
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
