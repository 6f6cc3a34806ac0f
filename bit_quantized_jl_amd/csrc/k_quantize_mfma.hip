// Dense QJL key quantization on the gfx950 matrix cores.
//
// Computes, for bfloat16 keys, Y = K S^T with v_mfma_f32_32x32x16_bf16
// (float32 accumulation; bf16 x bf16 products are exact), and fuses in
// registers: the sign test, packing of the signs into 32-bit words, and the
// key norm ||k||.  This is the key side of the QJL abstract (a JL projection
// whose coordinates are reduced to their signs) with a dense Gaussian S.
//
// Tiling.  A workgroup keeps the whole bf16 sketch in LDS (m*d*2 bytes: 64 KB
// at d=128, m=256) and its waves stream keys.  S is the MFMA A operand (rows
// are sketch coordinates), keys the B operand (columns): one wave owns 64 keys
// (two 32-key column tiles).  Each lane loads its key fragment straight from
// HBM: lane (c, h) = (lane % 32, lane / 32) holds half of the 16-byte chunks
// of key c (qm_chunk says which), and MFMA step t contracts one chunk from
// each lane half.  The contraction index is therefore a permutation of the key
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
//
// Schedule.  The W passes of a tile (one 32-coordinate tile each) run as
// T = d/16 MFMA steps; the S fragments stream from LDS through a ring of
// QM_RING registers refilled one step at a time, and, where registers allow,
// the sign bits of pass q - 1 are packed a few per step while pass q runs so
// that the VALU packing overlaps the matrix cores.  Bits and norms are
// written with non-temporal stores: a later kernel reads them, this one does
// not, and streaming them past the caches measured markedly faster.
//
// Short calls (decode-time appends) take quantize_small_kernel below, which
// forms the same sums without staging S in LDS.
#include <stdlib.h>
#include <string.h>

#include "device_common.h"
#include "mfma_image.h"

namespace qjl {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

namespace {

// A wave tile is RT 32-key column tiles: each S fragment read from LDS feeds
// RT MFMAs.  R S fragments are in flight from LDS at a time.

template <int T, int RT>
struct KeyTile {
  bf16x8_t a[RT][T];
};

// Load the B fragments of the 32 RT keys starting at k0.  Rows past n re-read
// row n-1 (their results are never stored): the loads stay unconditional, so
// the compiler can count them and wait only for the tile it needs.
template <int D, int RT>
__device__ __forceinline__ void load_tile(KeyTile<D / 16, RT> &kt, const uint16_t *__restrict__ K,
                                          int64_t k0, int64_t n, int r, int h) {
  constexpr int T = D / 16;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t row = k0 + 32 * rt + r;
    row = row < n ? row : n - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(K + row * D);
#pragma unroll
    for (int t = 0; t < T; ++t) kt.a[rt][t] = __builtin_bit_cast(bf16x8_t, src[qm_chunk(h, t)]);
  }
}

// S fragment number g of a tile walk: pass q = g / T covers coordinate tile
// tau = q ^ 1 (s = 1 before s = 0 within a word pair), step t = g % T.
template <int T>
__device__ __forceinline__ bf16x8_t s_fragment(const uint4 *sS, int g, int lane) {
  const int tau = (g / T) ^ 1, t = g % T;
  return __builtin_bit_cast(bf16x8_t, sS[(tau * T + t) * 64 + lane]);
}

// Shift the sign bits of acc[v1], acc[v1 - 1], ..., acc[v0] into x.
template <int V1, int V0>
__device__ __forceinline__ uint32_t pack_signs(uint32_t x, const floatx16_t &acc) {
#pragma unroll
  for (int v = V1; v >= V0; --v) x = __builtin_amdgcn_alignbit(x, __float_as_uint(acc[v]), 31);
  // Keep the packing here: left alone, the compiler sinks it to the stores
  // and every pass's accumulators stay live at once.
  asm volatile("" : "+v"(x));
  return x;
}

// Norms, projection, sign packing and stores for one wave tile of 32 RT keys.  With
// DEFER the bits of pass q - 1 are packed during pass q (one more pair of
// accumulators live); otherwise each pass is packed when it ends.  A
// scheduling barrier closes every MFMA step: without it the scheduler hoists
// all MFMAs of the tile and runs out of registers.  Norms of column tiles
// 2i and 2i + 1 leave in one 64-lane store (lane half h writes tile 2i + h).
template <int D, int M, int RT, int R, bool DEFER, bool MAPPED>
__device__ __forceinline__ void process_tile(const KeyTile<D / 16, RT> &kt, const uint4 *sS,
                                             int64_t k0, int64_t n, int lane, int r, int h,
                                             const RowMap &map, float *__restrict__ norms,
                                             uint32_t *__restrict__ bits) {
  constexpr int T = D / 16;
  constexpr int W = M / 32;
  constexpr int NF = W * T;    // S fragments per tile walk
  // The S reads below must stay inside the tile loop: hoisted out of it, all
  // m*d/512 fragments would be held in registers.
  asm volatile("" ::: "memory");
  bf16x8_t ring[R];
#pragma unroll
  for (int g = 0; g < R; ++g) ring[g] = s_fragment<T>(sS, g, lane);

  // Squared norms: each lane sums its half of the key, one chunk per MFMA
  // step of the first pass, in increasing chunk order.
  float ss[RT] = {};
  uint32_t zm[RT];

  uint32_t Wd[RT][W / 2];
  uint32_t x[RT] = {};
  floatx16_t prev[RT];
#pragma unroll
  for (int q = 0; q < W; ++q) {
    floatx16_t acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx16_t{};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int g = q * T + t;
      const bf16x8_t A = ring[g % R];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, kt.a[rt][t], acc[rt], 0, 0, 0);
      if (g + R < NF) ring[g % R] = s_fragment<T>(sS, g + R, lane);
      if (q == 0) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint4 v = __builtin_bit_cast(uint4, kt.a[rt][t]);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2_t kx = __builtin_bit_cast(bf16x2_t, w[e]);
            ss[rt] = __builtin_amdgcn_fdot2_f32_bf16(kx, kx, ss[rt], false);
          }
        }
      }
      if (DEFER && q > 0 && t > 0) {
        // Steps 1..T-1 pack the previous pass, registers 15 down to 0; step 0
        // would wait for that pass's last MFMA to finish writing them.
        constexpr int hi = 15;  // register packed first
        const int v1 = hi - (16 * (t - 1)) / (T - 1), v0 = hi + 1 - (16 * t) / (T - 1);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
          for (int v = 15; v >= 0; --v)
            if (v <= v1 && v >= v0)
              x[rt] = __builtin_amdgcn_alignbit(x[rt], __float_as_uint(prev[rt][v]), 31);
          asm volatile("" : "+v"(x[rt]));
        }
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    if (q == 0) {
      float nrm[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float tot = ss[rt] + __shfl_xor(ss[rt], 32);
        zm[rt] = tot > 0.f ? 0u : 0xFFFFFFFFu;
        nrm[rt] = sqrtf(tot);
      }
#pragma unroll
      for (int i = 0; i < RT / 2; ++i) {
        const int64_t key = k0 + 32 * (2 * i + h) + r;
        if (key < n)
          __builtin_nontemporal_store(h ? nrm[2 * i + 1] : nrm[2 * i],
                                      norms + (MAPPED ? map_row(map, key) : key));
      }
    }
    if (DEFER) {
      if (q > 0 && (q - 1) % 2 == 1) {  // pass q - 1 completed word (q - 1) / 2
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          Wd[rt][(q - 1) / 2] = ~x[rt] | zm[rt];
          x[rt] = 0;
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) prev[rt] = acc[rt];
    } else {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        x[rt] = pack_signs<15, 0>(x[rt], acc[rt]);
        if (q % 2 == 1) {
          Wd[rt][q / 2] = ~x[rt] | zm[rt];
          x[rt] = 0;
        }
      }
    }
  }
  if (DEFER) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      x[rt] = pack_signs<15, 0>(x[rt], prev[rt]);
      Wd[rt][W / 2 - 1] = ~x[rt] | zm[rt];
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t key = k0 + 32 * rt + r;
    if (key < n) {
      const int64_t row = MAPPED ? map_row(map, key) : key;
      if constexpr ((W / 2) % 4 == 0) {
        u32x4_t *dst = reinterpret_cast<u32x4_t *>(bits + row * W + h * (W / 2));
#pragma unroll
        for (int q = 0; q < W / 8; ++q)
          __builtin_nontemporal_store(
              u32x4_t{Wd[rt][4 * q], Wd[rt][4 * q + 1], Wd[rt][4 * q + 2], Wd[rt][4 * q + 3]},
              dst + q);
      } else {
        u32x2_t *dst = reinterpret_cast<u32x2_t *>(bits + row * W + h * (W / 2));
#pragma unroll
        for (int q = 0; q < W / 4; ++q)
          __builtin_nontemporal_store(u32x2_t{Wd[rt][2 * q], Wd[rt][2 * q + 1]}, dst + q);
      }
    }
  }
}

// Persistent kernel: each wave walks tiles of 32 RT keys with a stride of all
// waves in the grid; the grid is sized to what is resident at once.  Two
// waves per SIMD hide one another's HBM latency.  With PF a wave also issues
// the loads of its next tile before it processes the current one (two tiles'
// keys live in registers).
template <int D, int M, int WAVES, int RT, int R, bool DEFER, bool PF, bool MAPPED>
__global__ __launch_bounds__(64 * WAVES, 2) void quantize_mfma_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Simg, int64_t n, RowMap map,
    float *__restrict__ norms, uint32_t *__restrict__ bits) {
  static_assert(M % 128 == 0, "each lane stores whole 8-byte groups of words");
  __shared__ uint4 sS[M * D / 8];
  const int tid = threadIdx.x;
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(Simg);
    for (int i = tid; i < M * D / 8; i += 64 * WAVES) sS[i] = src[i];
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  constexpr int KEYS = 32 * RT;
  const int64_t ntiles = (n + KEYS - 1) / KEYS;
  const int64_t stride = (int64_t)gridDim.x * WAVES;
  int64_t tile = (int64_t)blockIdx.x * WAVES + wave;
  if constexpr (PF) {
    KeyTile<D / 16, RT> ka, kb;
    if (tile < ntiles) load_tile<D, RT>(ka, K, tile * KEYS, n, r, h);
    while (tile < ntiles) {
      const int64_t t1 = tile + stride;
      if (t1 < ntiles) load_tile<D, RT>(kb, K, t1 * KEYS, n, r, h);
      process_tile<D, M, RT, R, DEFER, MAPPED>(ka, sS, tile * KEYS, n, lane, r, h, map, norms,
                                               bits);
      if (t1 >= ntiles) break;
      const int64_t t2 = t1 + stride;
      if (t2 < ntiles) load_tile<D, RT>(ka, K, t2 * KEYS, n, r, h);
      process_tile<D, M, RT, R, DEFER, MAPPED>(kb, sS, t1 * KEYS, n, lane, r, h, map, norms,
                                               bits);
      tile = t2;
    }
  } else {
    for (; tile < ntiles; tile += stride) {
      KeyTile<D / 16, RT> kt;
      load_tile<D, RT>(kt, K, tile * KEYS, n, r, h);
      process_tile<D, M, RT, R, DEFER, MAPPED>(kt, sS, tile * KEYS, n, lane, r, h, map, norms,
                                               bits);
    }
  }
}

template <int D, int M, int WAVES, int RT, int R, bool DEFER, bool PF, bool MAPPED>
hipError_t launch_qm_kernel(const qjl_sketch *sk, const uint16_t *K, int64_t n,
                            const RowMap &map, float *norms, uint32_t *bits, hipStream_t st) {
  auto kern = quantize_mfma_kernel<D, M, WAVES, RT, R, DEFER, PF, MAPPED>;
  static PerDevice pd_res;  // workgroups resident on the whole device
  const int resident = per_device(pd_res, [&] { return resident_workgroups(kern, 64 * WAVES); });
  const int64_t ntiles = (n + 32 * RT - 1) / (32 * RT);
  const int64_t want = (ntiles + WAVES - 1) / WAVES;
  const int grid = (int)(want < resident ? want : resident);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WAVES), 0, st, K, sk->S16mfma, n, map, norms,
                     bits);
  return hipGetLastError();
}

// Launch shape per sketch size (measured on MI355X): up to m = 256 two
// 4-wave workgroups share a CU, each with its own copy of S, two column tiles
// per wave, four S fragments in flight, and packing deferred; at m = 512 S
// takes 128 KB of LDS, so one 8-wave workgroup per CU packs each pass as it
// ends to stay within two waves' registers per SIMD.
//
// Up to m = 256 the environment variable QJL_DENSE_SCHEDULE selects one of
// three other register schedules for unmapped launches (any other value, or
// none, keeps the one above).  All four form every sum from the same inputs
// in the same order and pack the same signs, so the bits and norms are
// identical; they differ only in time and power:
//   prefetch   the next tile's keys are loaded while the current one is
//              processed (two S fragments in flight, to fit the registers;
//              at d = m = 128 each pass packed as it ends)
//   rt4        four column tiles per wave (half the LDS reads of S), each
//              pass packed as it ends, two S fragments in flight
//   immediate  each pass packed as it ends (no deferral)
// On MI355X the default measured fastest; sustained, every schedule holds the
// socket at its power limit.
enum class QmSchedule { Default, Prefetch, Rt4, Immediate };

QmSchedule dense_schedule() {
  const char *s = getenv("QJL_DENSE_SCHEDULE");
  if (s == nullptr) return QmSchedule::Default;
  if (strcmp(s, "prefetch") == 0) return QmSchedule::Prefetch;
  if (strcmp(s, "rt4") == 0) return QmSchedule::Rt4;
  if (strcmp(s, "immediate") == 0) return QmSchedule::Immediate;
  return QmSchedule::Default;
}

template <int D, int M, bool MAPPED>
hipError_t launch_qm(const qjl_sketch *sk, const uint16_t *K, int64_t n, const RowMap &map,
                     float *norms, uint32_t *bits, hipStream_t st) {
  if constexpr (M <= 256 && !MAPPED) {
    switch (dense_schedule()) {
      case QmSchedule::Prefetch: {
        constexpr bool PDEFER = !(D == 128 && M == 128);  // there deferral would spill
        return launch_qm_kernel<D, M, 4, 2, 2, PDEFER, true, false>(sk, K, n, map, norms, bits,
                                                                    st);
      }
      case QmSchedule::Rt4:
        return launch_qm_kernel<D, M, 4, 4, 2, false, false, false>(sk, K, n, map, norms, bits,
                                                                     st);
      case QmSchedule::Immediate:
        return launch_qm_kernel<D, M, 4, 2, 4, false, false, false>(sk, K, n, map, norms, bits,
                                                                     st);
      case QmSchedule::Default:
        break;
    }
  }
  constexpr int WAVES = M <= 256 ? 4 : 8;
  constexpr bool DEFER = M <= 256;
  return launch_qm_kernel<D, M, WAVES, 2, 4, DEFER, false, MAPPED>(sk, K, n, map, norms, bits,
                                                                   st);
}

// Few keys (a decode-time append of one key per head): the same sums with
// the operand image read from global memory instead of staged in LDS, one
// wave per (32 keys, output word pair p).  Lane (r, h) forms tiles 2p + 1
// and 2p (coordinates of word p + h W/2 of key r), in the quantizer's order:
// the same MFMA inputs accumulated in the same order, the same sign packing
// and the same norm chain, so the bits and norms equal the quantizer's.
template <int D, bool MAPPED>
__global__ __launch_bounds__(256) void quantize_small_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Simg, int m, int64_t n,
    RowMap map, float *__restrict__ norms, uint32_t *__restrict__ bits) {
  constexpr int T = D / 16;
  const int lane = threadIdx.x & 63;
  const int p = blockIdx.y * 4 + (threadIdx.x >> 6);  // word pair
  const int W = m / 32;
  if (p >= W / 2) return;
  const int r = lane & 31, h = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x * 32 + r;
  const int64_t lrow = row < n ? row : n - 1;  // rows past n re-read row n - 1, store nothing
  const uint4 *src = reinterpret_cast<const uint4 *>(K + lrow * D);
  const uint4 *img = reinterpret_cast<const uint4 *>(Simg) + lane;
  bf16x8_t ka[T], s1[T], s0[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    ka[t] = __builtin_bit_cast(bf16x8_t, src[qm_chunk(h, t)]);
    s1[t] = __builtin_bit_cast(bf16x8_t, img[((2 * p + 1) * T + t) * 64]);
    s0[t] = __builtin_bit_cast(bf16x8_t, img[((2 * p) * T + t) * 64]);
  }
  floatx16_t acc1 = floatx16_t{}, acc0 = floatx16_t{};
  float ss = 0.f;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s1[t], ka[t], acc1, 0, 0, 0);
    const uint4 v = __builtin_bit_cast(uint4, ka[t]);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2_t kx = __builtin_bit_cast(bf16x2_t, w[e]);
      ss = __builtin_amdgcn_fdot2_f32_bf16(kx, kx, ss, false);
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t)
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s0[t], ka[t], acc0, 0, 0, 0);
  const float tot = ss + __shfl_xor(ss, 32);
  const uint32_t zm = tot > 0.f ? 0u : 0xFFFFFFFFu;
  uint32_t x = pack_signs<15, 0>(0u, acc1);
  x = pack_signs<15, 0>(x, acc0);
  if (row < n) {
    const int64_t orow = MAPPED ? map_row(map, row) : row;
    bits[orow * W + p + h * (W / 2)] = ~x | zm;
    if (p == 0 && h == 0) norms[orow] = sqrtf(tot);
  }
}

template <int D, bool MAPPED>
hipError_t launch_qs(const qjl_sketch *sk, const uint16_t *K, int64_t n, const RowMap &map,
                     float *norms, uint32_t *bits, hipStream_t st) {
  const int W = sk->host.m / 32;
  const dim3 grid((unsigned)((n + 31) / 32), (unsigned)((W / 2 + 3) / 4));
  hipLaunchKernelGGL((quantize_small_kernel<D, MAPPED>), grid, dim3(256), 0, st, K, sk->S16mfma,
                     sk->host.m, n, map, norms, bits);
  return hipGetLastError();
}

template <bool MAPPED>
hipError_t launch_qm_dm(const qjl_sketch *sk, const uint16_t *K, int64_t n, const RowMap &map,
                        float *norms, uint32_t *bits, hipStream_t st) {
  const int d = sk->host.d, m = sk->host.m;
  if (d == 128 && m == 128) return launch_qm<128, 128, MAPPED>(sk, K, n, map, norms, bits, st);
  if (d == 128 && m == 256) return launch_qm<128, 256, MAPPED>(sk, K, n, map, norms, bits, st);
  if (d == 128 && m == 512) return launch_qm<128, 512, MAPPED>(sk, K, n, map, norms, bits, st);
  if (d == 64 && m == 128) return launch_qm<64, 128, MAPPED>(sk, K, n, map, norms, bits, st);
  if (d == 64 && m == 256) return launch_qm<64, 256, MAPPED>(sk, K, n, map, norms, bits, st);
  if (d == 64 && m == 512) return launch_qm<64, 512, MAPPED>(sk, K, n, map, norms, bits, st);
  return hipErrorInvalidValue;
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

hipError_t launch_quantize_mfma(const qjl_sketch *sk, const void *Kv, int64_t n, const RowMap &map,
                                float *norms, uint32_t *bits, hipStream_t st) {
  const uint16_t *K = static_cast<const uint16_t *>(Kv);
#ifndef QJL_QS_MAX
#define QJL_QS_MAX 16384
#endif
  if (n <= QJL_QS_MAX) {  // latency-bound: skip staging S in LDS
    const bool mp = map.per_group != 0;
    if (sk->host.d == 128)
      return mp ? launch_qs<128, true>(sk, K, n, map, norms, bits, st)
                : launch_qs<128, false>(sk, K, n, map, norms, bits, st);
    return mp ? launch_qs<64, true>(sk, K, n, map, norms, bits, st)
              : launch_qs<64, false>(sk, K, n, map, norms, bits, st);
  }
  if (map.per_group != 0) return launch_qm_dm<true>(sk, K, n, map, norms, bits, st);
  return launch_qm_dm<false>(sk, K, n, map, norms, bits, st);
}

}  // namespace qjl
