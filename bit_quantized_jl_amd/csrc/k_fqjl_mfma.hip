// FQJL key quantization with its first stage on the gfx950 matrix cores
// ("Fast Quantized Johnson-Lindenstrauss Transforms" page: block b of the
// sketch is H diag(G_b) Pi_b (H/sqrt d) diag(D_b), optional Gaussian dither
// before the sign).
//
// For bfloat16 keys, everything before the Gaussian diagonal is one matrix
// with entries +-1:  M_b = Pi_b H diag(D_b), M_b[i][c] = H[P_b[i]][c] D_b[c]
// (the 1/sqrt d lives in the stored G_b / sqrt d; the image also carries
// the sign of G_b[i] in row i, and the kernel scales by |G_b[i]| / sqrt d,
// which keeps -0 out of the rest of the chain).  Its products with bf16
// key elements are exact and the matrix cores sum them in float32, so
// u_b = M_b k comes out of v_mfma_f32_32x32x16_bf16 exactly as from the
// butterfly network, up to the order of the float32 additions.  What
// remains runs on the vector ALUs per key: z = (G_b / sqrt d) * u_b, the
// second Walsh-Hadamard transform y = H z, the dither, the sign and the
// packing -- half the vector work of the all-butterfly kernel.
//
// Layout.  The operand image of [M_0; M_1; ...] uses the dense quantizer's
// order (mfma_image.h) with one difference in the row order: tile
// tau = 4 b + p (block b, pass p) puts coordinate 64 h + 16 p + v of block b
// in accumulator register v of lane half h.  So after the four passes of a
// block, lane (key r, half h) holds u_b[64 h .. 64 h + 63] of its key, in
// order, in its 64 accumulator registers.  The second transform splits as
// H_128 = [[H_64, H_64], [H_64, -H_64]]: each lane half runs H_64 on its own
// half (a_h); one v_permlane32_swap per coordinate pair (i, i + 32) gives
// half h a_0 and a_1 at coordinate i + 32 h, and it keeps both
// y[32 h + i] = a_0 + a_1 and y[64 + 32 h + i] = a_0 - a_1.  Those are
// output words 4 b + h and 4 b + 2 + h; one more swap per word pair puts
// them in row order for the store.
//
// Schedule as in the dense quantizer: S fragments stream from LDS through a
// ring of registers, each feeding RT column tiles of 32 keys; the key tile is
// loaded straight into MFMA operand registers, one tile ahead; the norm is
// summed with v_dot2c_f32_bf16 during the first pass.  Two waves per SIMD
// hide one another's vector work behind the matrix cores.  (Measured on the
// 7B shape: the prefetch gains 2-3%; two column tiles per wave spill and lose
// 25%; alternating the four passes' accumulation chains changes nothing.)
//
// Three kernels share the layout: fqjl_mfma_kernel (persistent, image in
// LDS: large calls), fqjl_mfma_small_kernel (short calls at m >= 256, image
// fragments from L2, one wave per key tile and block) and
// fqjl_project_mfma_kernel (queries: the same first and second stage, the
// float32 values stored instead of signs).  All three form the same sums
// in the same order, so a key's bits do not depend on the call's size and
// a projected key has the signs of its bits.
#include "device_common.h"
#include "fwht_common.h"
#include "mfma_image.h"

namespace qjl {

namespace {

// Sign bits of 32 consecutive coordinates, bit t = [u[t] >= 0], one
// v_alignbit_b32 each.  No -0 reaches here, so the sign bit alone decides:
// the matrix cores start from +0 and return +0 for an all-zero sum, the
// Gaussian diagonal's signs sit in the image (|G| > 0 multiplies), so z has
// no -0; and a butterfly or a dither add yields -0 only from -0 operands
// (x + (-x) rounds to +0).  A zero key thus packs to all ones.
__device__ __forceinline__ uint32_t pack_signs(const float *u) {
  uint32_t word = 0;
#pragma unroll
  for (int t = 31; t >= 0; --t) word = __builtin_amdgcn_alignbit(word, __float_as_uint(u[t]), 31);
  return ~word;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int FM_RING = 4;  // S fragments in flight from LDS


template <int T, int RT>
struct FmKeys {
  bf16x8_t a[RT][T];
};

// The B fragments of the 32 RT keys from k0 (rows past n re-read row n - 1;
// their results are never stored), as the dense quantizer loads them.
template <int T, int RT>
__device__ __forceinline__ void fm_load(FmKeys<T, RT> &kt, const uint16_t *__restrict__ K,
                                        int64_t k0, int64_t n, int r, int h) {
  constexpr int D = 16 * T;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t row = k0 + 32 * rt + r;
    row = row < n ? row : n - 1;
    const uint4 *src = reinterpret_cast<const uint4 *>(K + row * D);
#pragma unroll
    for (int t = 0; t < T; ++t) kt.a[rt][t] = __builtin_bit_cast(bf16x8_t, src[qm_chunk(h, t)]);
  }
}

// The dither of the coordinates a lane half holds after the second stage of
// block b (z[0 .. 31]: sign word 4 b + h of the key, z[32 .. 63]: word
// 4 b + 2 + h; a128: the magnitudes of block b's 128 coordinates).  Lane half
// h draws word 2 b + h of the key's signs (sign words 4 b + 2 h and
// 4 b + 2 h + 1), and one swap hands half 0 the high halves of the two
// draws (words 4 b, 4 b + 2) and half 1 the low halves (4 b + 1, 4 b + 3).
template <int M>
__device__ __forceinline__ void fm_dither(float (&z)[64], int b, int h, float amp, uint64_t dkey,
                                          int64_t key_index, const float *a128) {
  const uint64_t dw = dither_draw(dkey, (uint64_t)key_index, M, 2 * b + h);
  const auto sw =
      __builtin_amdgcn_permlane32_swap((uint32_t)(dw >> 32), (uint32_t)dw, false, false);
  dither_add<32>(&z[0], amp, sw[0], 0, a128 + 32 * h);
  dither_add<32>(&z[32], amp, sw[1], 0, a128 + 64 + 32 * h);
}

template <int M, int WAVES, int RT, bool DITHER, bool MAPPED>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void fqjl_mfma_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Fimg,
    const float *__restrict__ Gs, int64_t n, int64_t base, RowMap map, float rho, uint64_t dkey,
    const float *__restrict__ Dmag, float *__restrict__ norms, uint32_t *__restrict__ bits) {
  constexpr int D = 128, T = D / 16, NB = M / D, W = M / 32;
  constexpr int NF = NB * 4 * T;  // S fragments per tile walk
  constexpr int R = FM_RING;
  __shared__ uint4 sF[M * D / 8];
  __shared__ float sG[M];
  __shared__ float sA[DITHER ? M : 1];  // dither magnitudes
  const int tid = threadIdx.x;
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(Fimg);
    for (int i = tid; i < M * D / 8; i += 64 * WAVES) sF[i] = src[i];
    for (int i = tid; i < M; i += 64 * WAVES) sG[i] = fabsf(Gs[i]);
    if constexpr (DITHER)
      for (int i = tid; i < M; i += 64 * WAVES) sA[i] = Dmag[i];
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 31, h = lane >> 5;
  constexpr int KEYS = 32 * RT;
  const int64_t ntiles = (n + KEYS - 1) / KEYS;
  const int64_t stride = (int64_t)gridDim.x * WAVES;
  // Up to m = 256 the next tile's keys load while this one is processed
  // (rows past n are clamped, so a wave's last prefetch reads row n - 1 and
  // is discarded); at m = 512 the registers are not there.
  constexpr bool PF = M <= 256;
  FmKeys<T, RT> nxt;
  if (PF) fm_load<T, RT>(nxt, K, ((int64_t)blockIdx.x * WAVES + wave) * KEYS, n, r, h);
  for (int64_t tile = (int64_t)blockIdx.x * WAVES + wave; tile < ntiles; tile += stride) {
    const int64_t k0 = tile * KEYS;
    FmKeys<T, RT> kt;
    if (PF) {
      kt = nxt;
      fm_load<T, RT>(nxt, K, (tile + stride) * KEYS, n, r, h);
    } else {
      fm_load<T, RT>(kt, K, k0, n, r, h);
    }
    // The fragment reads must stay inside the tile loop: hoisted, all of the
    // image would be held in registers.
    asm volatile("" ::: "memory");
    bf16x8_t ring[R];
#pragma unroll
    for (int g = 0; g < R; ++g) ring[g] = __builtin_bit_cast(bf16x8_t, sF[g * 64 + lane]);
    float ss[RT] = {};
    float nrm[RT];
    uint32_t held[RT][2];  // the previous (even) block's two words, see the stores
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      // The wave issuing its matrix-core chain runs at a raised priority and
      // drops it for the vector epilogue, so the other wave's epilogue fills
      // the gaps without delaying the chain: 212 against 231 us at m = 256,
      // 406 against 427 us at m = 512; with dither 261 against 267 us.
      __builtin_amdgcn_s_setprio(1);
      floatx16_t acc[RT][4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt][p] = floatx16_t{};
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const int g = (4 * b + p) * T + t;
          const bf16x8_t A = ring[g % R];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
            acc[rt][p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, kt.a[rt][t], acc[rt][p], 0, 0, 0);
          if (g + R < NF) ring[g % R] = __builtin_bit_cast(bf16x8_t, sF[(g + R) * 64 + lane]);
          if (b == 0 && p == 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              const uint4 v = __builtin_bit_cast(uint4, kt.a[rt][t]);
              const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bf16x2_t kx = __builtin_bit_cast(bf16x2_t, w4[e]);
                ss[rt] = __builtin_amdgcn_fdot2_f32_bf16(kx, kx, ss[rt], false);
              }
            }
          }
          asm volatile("" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (b == 0) {
        // each lane summed half of its key's chunks; lane half h stores the
        // norm of column tile h (for RT = 1, half 0 stores)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) nrm[rt] = sqrtf(ss[rt] + __shfl_xor(ss[rt], 32));
        if (RT > 1 || h == 0) {
          const int64_t key = k0 + 32 * (RT > 1 ? h : 0) + r;
          if (key < n)
            __builtin_nontemporal_store(RT > 1 && h ? nrm[RT > 1 ? 1 : 0] : nrm[0],
                                        norms + (MAPPED ? map_row(map, key) : key));
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // ---- second stage of block b, per column tile
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float z[64];
        const float4 *gp = reinterpret_cast<const float4 *>(sG + 128 * b + 64 * h);
        // z = |G_b| u with the first butterfly stage (pairs 2i, 2i + 1)
        // fused in: one multiply and two fused multiply-adds per pair
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float4 gv = gp[k];
          const float g4[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float ua = acc[rt][k / 4][4 * (k % 4) + e];
            const float t = acc[rt][k / 4][4 * (k % 4) + e + 1] * g4[e + 1];
            z[4 * k + e] = fmaf(ua, g4[e], t);
            z[4 * k + e + 1] = fmaf(ua, g4[e], -t);
          }
        }
        fwht_reg<64, 2>(z);
        // Top stage across the lane halves, two coordinates (i, i + 32) at a
        // time: one swap brings a_0 and a_1 of coordinate i to half 0 and of
        // i + 32 to half 1, and each half keeps both the sum and the
        // difference.  Lane half h then holds y[32 h + i] in z[i] and
        // y[64 + 32 h + i] in z[32 + i]: its words are 4 b + h and
        // 4 b + 2 + h, put in row order by one swap per word pair below.
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[i]),
                                                           __float_as_uint(z[i + 32]), false, false);
          const float x = __uint_as_float(p1[0]), y = __uint_as_float(p1[1]);
          z[i] = x + y;
          z[i + 32] = x - y;
        }
        const int64_t key = k0 + 32 * rt + r;
        const int64_t orow = MAPPED ? map_row(map, key < n ? key : 0) : (key < n ? key : 0);
        if (DITHER) fm_dither<M>(z, b, h, rho * nrm[rt], dkey, base + orow, sA + 128 * b);
        const uint32_t w0 = pack_signs(&z[0]), w1 = pack_signs(&z[32]);
        if constexpr (NB != 2) {
          // One swap gives lane half h words 4 b + 2 h and 4 b + 2 h + 1.
          // m = 128: a row is 16 bytes, written by the two halves in one
          // instruction; m = 512 keeps 8-byte writes (no registers to spare)
          const auto sw = __builtin_amdgcn_permlane32_swap(w0, w1, false, false);
          if (key < n)
            __builtin_nontemporal_store(
                u32x2_t{sw[0], sw[1]}, reinterpret_cast<u32x2_t *>(bits + orow * W + 4 * b + 2 * h));
        } else if (b % 2 == 0) {
          held[rt][0] = w0;  // words 4b + h and 4b + 2 + h: written with the next block's
          held[rt][1] = w1;
        } else {
          // Blocks b - 1 and b hold words [4 (b - 1), 4 b + 4) of the row, two
          // per lane.  One swap per register gives lane half 0 the four words
          // of block b - 1 and half 1 those of block b, so each half stores 16
          // contiguous bytes and the pair of halves the whole 32-byte span
          // (split 8-byte writes made the caches fetch the lines first).
          const auto s0 = __builtin_amdgcn_permlane32_swap(held[rt][0], w0, false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(held[rt][1], w1, false, false);
          if (key < n)
            __builtin_nontemporal_store(
                u32x4_t{s0[0], s0[1], s1[0], s1[1]},
                reinterpret_cast<u32x4_t *>(bits + orow * W + 4 * (b - 1) + 4 * h));
        }
        // keep the next block's matrix work (and its registers) out of this one
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// The short-call kernel's second stage of block b for one key, in two parts
// (the output row is formed between them).  The arithmetic is that of
// fqjl_mfma_kernel's epilogue, operation for operation, which keeps the
// two kernels' bits identical; that kernel keeps its own copy, since at its
// 256-register limit the inlined helpers spill.
// fm_transform: z = |G_b| * u (gp: this lane half's 64 values of
// |G_b| / sqrt d), then y = H z: H_64 per lane half (its first stage fused
// with the scaling, as in fqjl_mfma_kernel) and the top stage across the
// halves; afterwards lane half h holds y[64 h .. 64 h + 63].
__device__ __forceinline__ void fm_transform(const floatx16_t (&acc)[4], const float4 *gp,
                                             float (&z)[64]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float4 gv = gp[k];
    const float g4[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float ua = acc[k / 4][4 * (k % 4) + e];
      const float t = acc[k / 4][4 * (k % 4) + e + 1] * g4[e + 1];
      z[4 * k + e] = fmaf(ua, g4[e], t);
      z[4 * k + e + 1] = fmaf(ua, g4[e], -t);
    }
  }
  fwht_reg<64, 2>(z);
  // Top stage, two coordinates (i, i + 32) at a time: one swap brings a_0
  // and a_1 of coordinate i to half 0 and of i + 32 to half 1, and each half
  // keeps both the sum and the difference: lane half h then holds
  // y[32 h + i] in z[i] and y[64 + 32 h + i] in z[32 + i].
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const auto p1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(z[i]),
                                                     __float_as_uint(z[i + 32]), false, false);
    const float x = __uint_as_float(p1[0]), y = __uint_as_float(p1[1]);
    z[i] = x + y;
    z[i + 32] = x - y;
  }
}

// fm_finish: dither of size amp for key drow (a128: block b's magnitudes),
// sign, and the two words: 4 b + h and 4 b + 2 + h of the row.
template <int M, bool DITHER>
__device__ __forceinline__ void fm_finish(float (&z)[64], int b, int h, float amp, uint64_t dkey,
                                          int64_t drow, const float *a128, uint32_t &w0,
                                          uint32_t &w1) {
  if (DITHER) fm_dither<M>(z, b, h, amp, dkey, drow, a128);
  w0 = pack_signs(&z[0]);
  w1 = pack_signs(&z[32]);
}

// Short calls (decode-time appends, m >= 256): one wave per 32 keys and
// block b, the block's 32 image fragments read from global memory (L2)
// instead of staging the whole image in LDS, and the blocks of a key on
// different waves.  Measured per call at m = 256: 7.8 us against 10.2 us
// for 256 keys.  From ~64K keys on, the persistent kernel is as
// fast or faster (at the 7B shape 242 against 512 us).  Same key fragments,
// the same matrix-core accumulations in the same order, the same norm chain
// and the same second stage as fqjl_mfma_kernel, so the bits and norms are
// those of that kernel; a cache filled by appends equals one quantized in a
// single call.
template <int M, bool DITHER, bool MAPPED>
__global__ __launch_bounds__(64) void fqjl_mfma_small_kernel(
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ Fimg,
    const float *__restrict__ Gs, int64_t n, int64_t base, RowMap map, float rho, uint64_t dkey,
    const float *__restrict__ Dmag, float *__restrict__ norms, uint32_t *__restrict__ bits) {
  constexpr int D = 128, T = D / 16, W = M / 32;
  __shared__ float sG[D];
  __shared__ float sA[DITHER ? D : 1];  // block b's dither magnitudes
  const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
  const int b = blockIdx.y;
  sG[lane] = fabsf(Gs[D * b + lane]);
  sG[lane + 64] = fabsf(Gs[D * b + lane + 64]);
  if constexpr (DITHER) {
    sA[lane] = Dmag[D * b + lane];
    sA[lane + 64] = Dmag[D * b + lane + 64];
  }
  const int64_t k0 = (int64_t)blockIdx.x * 32;
  FmKeys<T, 1> kt;
  fm_load<T, 1>(kt, K, k0, n, r, h);
  const uint4 *img = reinterpret_cast<const uint4 *>(Fimg) + (size_t)4 * b * T * 64 + lane;
  floatx16_t acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    acc[p] = floatx16_t{};
#pragma unroll
    for (int t = 0; t < T; ++t)
      acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, img[(p * T + t) * 64]), kt.a[0][t], acc[p], 0, 0, 0);
  }
  float ss = 0.f;
  if (DITHER || b == 0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint4 v = __builtin_bit_cast(uint4, kt.a[0][t]);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t kx = __builtin_bit_cast(bf16x2_t, w4[e]);
        ss = __builtin_amdgcn_fdot2_f32_bf16(kx, kx, ss, false);
      }
    }
  }
  const float nrm = sqrtf(ss + __shfl_xor(ss, 32));
  const int64_t key = k0 + r;
  const int64_t orow = MAPPED ? map_row(map, key < n ? key : 0) : (key < n ? key : 0);
  if (b == 0 && h == 0 && key < n) __builtin_nontemporal_store(nrm, norms + orow);
  __syncthreads();
  float z[64];
  fm_transform(acc, reinterpret_cast<const float4 *>(sG + 64 * h), z);
  uint32_t w0, w1;
  fm_finish<M, DITHER>(z, b, h, DITHER ? rho * nrm : 0.f, dkey, base + orow, sA, w0, w1);
  const auto sw = __builtin_amdgcn_permlane32_swap(w0, w1, false, false);  // words 4b + 2h, +1
  if (key < n)
    __builtin_nontemporal_store(u32x2_t{sw[0], sw[1]},
                                reinterpret_cast<u32x2_t *>(bits + orow * W + 4 * b + 2 * h));
}

// Query projection y = S q of bf16 queries (no dither, no sign), laid out
// as the short-call quantizer: one wave per 32 queries and block b; lane
// half h writes the 64 coordinates fm_transform leaves it, two runs of 128
// contiguous bytes.
// The matrix cores' sums are exact products summed in float32, so y equals
// the quantizer's pre-sign values for the same vector: a bf16 key projected
// as a query has the signs of its quantized bits (rho = 0).
template <int M>
__global__ __launch_bounds__(64) void fqjl_project_mfma_kernel(const uint16_t *__restrict__ Q,
                                                               const uint16_t *__restrict__ Fimg,
                                                               const float *__restrict__ Gs,
                                                               int64_t n, float *__restrict__ Y) {
  constexpr int D = 128, T = D / 16;
  __shared__ float sG[D];
  const int lane = threadIdx.x, r = lane & 31, h = lane >> 5;
  const int b = blockIdx.y;
  sG[lane] = fabsf(Gs[D * b + lane]);
  sG[lane + 64] = fabsf(Gs[D * b + lane + 64]);
  const int64_t q0 = (int64_t)blockIdx.x * 32;
  FmKeys<T, 1> kt;
  fm_load<T, 1>(kt, Q, q0, n, r, h);
  const uint4 *img = reinterpret_cast<const uint4 *>(Fimg) + (size_t)4 * b * T * 64 + lane;
  floatx16_t acc[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    acc[p] = floatx16_t{};
#pragma unroll
    for (int t = 0; t < T; ++t)
      acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, img[(p * T + t) * 64]), kt.a[0][t], acc[p], 0, 0, 0);
  }
  __syncthreads();
  float z[64];
  fm_transform(acc, reinterpret_cast<const float4 *>(sG + 64 * h), z);
  const int64_t q = q0 + r;
  if (q < n) {  // coordinates 128 b + 32 h + [0, 32) and 128 b + 64 + 32 h + [0, 32)
    float4 *lo = reinterpret_cast<float4 *>(Y + q * M + 128 * b + 32 * h);
    float4 *hi = reinterpret_cast<float4 *>(Y + q * M + 128 * b + 64 + 32 * h);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lo[k] = make_float4(z[4 * k], z[4 * k + 1], z[4 * k + 2], z[4 * k + 3]);
      hi[k] = make_float4(z[32 + 4 * k], z[33 + 4 * k], z[34 + 4 * k], z[35 + 4 * k]);
    }
  }
}

template <int M, bool DITHER, bool MAPPED>
hipError_t launch_fm(const qjl_sketch *sk, const uint16_t *K, int64_t n, int64_t base,
                     const RowMap &map, float *norms, uint32_t *bits, hipStream_t st) {
#ifndef QJL_FM_RT
#define QJL_FM_RT 1
#endif
#ifndef QJL_FS_MAX
#define QJL_FS_MAX 16384
#endif
  // Latency-bound calls skip staging the image in LDS (m = 128 has a
  // single block per key, which the persistent kernel serves as fast).
  if (M >= 256 && n <= QJL_FS_MAX) {
    const dim3 grid((unsigned)((n + 31) / 32), M / 128);
    hipLaunchKernelGGL((fqjl_mfma_small_kernel<M, DITHER, MAPPED>), grid, dim3(64), 0, st, K,
                       sk->Fmfma, sk->Gs, n, base, map, sk->host.rho, sk->dither_key, sk->Dmag,
                       norms, bits);
    return hipGetLastError();
  }
  constexpr int RT = QJL_FM_RT;
  // two 4-wave workgroups per compute unit, or one of 8 waves where the
  // image (m = 512) leaves LDS for one
  constexpr int WAVES = M <= 256 ? 4 : 8;
  auto kern = fqjl_mfma_kernel<M, WAVES, RT, DITHER, MAPPED>;
  static PerDevice pd_res;  // workgroups resident on the whole device
  const int resident = per_device(pd_res, [&] { return resident_workgroups(kern, 64 * WAVES); });
  const int64_t ntiles = (n + 32 * RT - 1) / (32 * RT);
  const int64_t want = (ntiles + WAVES - 1) / WAVES;
  const int grid = (int)(want < resident ? want : resident);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * WAVES), 0, st, K, sk->Fmfma, sk->Gs, n, base,
                     map, sk->host.rho, sk->dither_key, sk->Dmag, norms, bits);
  return hipGetLastError();
}

template <int M>
hipError_t launch_fm_m(const qjl_sketch *sk, const uint16_t *K, int64_t n, int64_t base,
                       const RowMap &map, float *norms, uint32_t *bits, hipStream_t st) {
  const bool dith = sk->host.rho > 0.f, mapped = map.per_group != 0;
  if (dith && mapped) return launch_fm<M, true, true>(sk, K, n, base, map, norms, bits, st);
  if (dith) return launch_fm<M, true, false>(sk, K, n, base, map, norms, bits, st);
  if (mapped) return launch_fm<M, false, true>(sk, K, n, base, map, norms, bits, st);
  return launch_fm<M, false, false>(sk, K, n, base, map, norms, bits, st);
}

}  // namespace

bool fqjl_mfma_supported(const qjl_sketch *sk, const void *K, int dtype, const uint32_t *bits) {
  const HostSketch &h = sk->host;
  if (h.variant == QJL_VARIANT_DENSE || dtype != QJL_DTYPE_BF16 || sk->Fmfma == nullptr)
    return false;
  if (!fqjl_mfma_image_shape(h.d, h.m)) return false;
  return ((uintptr_t)K & 15) == 0 && ((uintptr_t)bits & 15) == 0;
}

bool fqjl_project_mfma_supported(const qjl_sketch *sk, const void *q, int dtype, const float *Y) {
  const HostSketch &h = sk->host;
  if (h.variant == QJL_VARIANT_DENSE || dtype != QJL_DTYPE_BF16 || sk->Fmfma == nullptr)
    return false;
  if (!fqjl_mfma_image_shape(h.d, h.m)) return false;
  return ((uintptr_t)q & 15) == 0 && ((uintptr_t)Y & 15) == 0;
}

hipError_t launch_fqjl_project_mfma(const qjl_sketch *sk, const void *q, int64_t n, float *Y,
                                    hipStream_t st) {
  const uint16_t *Q = static_cast<const uint16_t *>(q);
  if ((n + 31) / 32 > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + 31) / 32), sk->host.m / 128);
  switch (sk->host.m) {
    case 128:
      hipLaunchKernelGGL(fqjl_project_mfma_kernel<128>, grid, dim3(64), 0, st, Q, sk->Fmfma,
                         sk->Gs, n, Y);
      break;
    case 256:
      hipLaunchKernelGGL(fqjl_project_mfma_kernel<256>, grid, dim3(64), 0, st, Q, sk->Fmfma,
                         sk->Gs, n, Y);
      break;
    case 512:
      hipLaunchKernelGGL(fqjl_project_mfma_kernel<512>, grid, dim3(64), 0, st, Q, sk->Fmfma,
                         sk->Gs, n, Y);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fqjl_mfma(const qjl_sketch *sk, const void *Kv, int64_t n, int64_t base,
                            const RowMap &map, float *norms, uint32_t *bits, hipStream_t st) {
  const uint16_t *K = static_cast<const uint16_t *>(Kv);
  switch (sk->host.m) {
    case 128: return launch_fm_m<128>(sk, K, n, base, map, norms, bits, st);
    case 256: return launch_fm_m<256>(sk, K, n, base, map, norms, bits, st);
    case 512: return launch_fm_m<512>(sk, K, n, base, map, norms, bits, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qjl
