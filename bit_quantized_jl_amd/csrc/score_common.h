// Shared device code of the matrix-core score path (the score kernel and the
// fused decode-attention kernel): the query held exactly as fp8 limbs, and the
// per-tile MFMA sum.  The encoding is described at the top of k_score_mfma.hip.
#pragma once

#include "device_common.h"

namespace qjl {
namespace sc {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int SM_THREADS = 256;
constexpr int SM_WAVES = 4;

// e4m3 bit pattern of an integer |v| <= 64 with at most 4 significant bits:
// such a value is exact in float32, whose sign, exponent (rebased from 127 to
// 7) and top three mantissa bits are the e4m3 fields.
__device__ __forceinline__ uint32_t e4m3_of_int(int v) {
  const uint32_t f = __float_as_uint((float)v);
  const uint32_t mag = ((f >> 20) & 0x7FFu) - (120u << 3);
  return v == 0 ? 0u : (((f >> 24) & 0x80u) | (mag & 0x7Fu));
}

// Wavefront reductions with DPP: row_shr 1, 2, 4, 8 fold each 16-lane row
// into its lane 15, row_bcast 15 and 31 fold the rows into lane 63, which is
// then read as a scalar.  Lanes without a DPP source keep the identity.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWMASK, 0xf, false);
}
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);  // v >= 0: max on floats, identity 0
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x111, 0xf>(0, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x112, 0xf>(0, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x114, 0xf>(0, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x118, 0xf>(0, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x142, 0xa>(0, x))));
  x = __float_as_int(fmaxf(__int_as_float(x), __int_as_float(dpp<0x143, 0xc>(0, x))));
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ int wave_sum(int x) {
  x += dpp<0x111, 0xf>(0, x);
  x += dpp<0x112, 0xf>(0, x);
  x += dpp<0x114, 0xf>(0, x);
  x += dpp<0x118, 0xf>(0, x);
  x += dpp<0x142, 0xa>(0, x);
  x += dpp<0x143, 0xc>(0, x);
  return __builtin_amdgcn_readlane(x, 63);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(n) leaving the other counters unconstrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data only.  __syncthreads() also fences global
// memory, which would wait for every ring DMA in flight; LDS writes of a wave
// are complete once its lgkmcnt drains.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

typedef __attribute__((address_space(3))) unsigned char lds_u8_t;
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return (uint32_t)(uintptr_t)((const lds_u8_t *)p);
}

// Query values of the NQ queries of one pass (rows q0 .. q0 + nqp - 1 at
// Sq_q0): lane l holds coordinates l + 64 b.  A slot past nqp reads query 0
// and is zeroed, so every load is unconditional (the compiler can count them).
template <int M, int NQ>
__device__ __forceinline__ void load_query_values(const float *__restrict__ Sq_q0, int nqp,
                                                  int lane, float (&sv)[NQ][M / 64]) {
  static_assert(M % 64 == 0, "whole coordinate blocks per lane");
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    const float *src = Sq_q0 + (qi < nqp ? qi : 0) * (int64_t)M;
#pragma unroll
    for (int b = 0; b < M / 64; ++b) {
      const float v = src[lane + 64 * b];
      sv[qi][b] = qi < nqp ? v : 0.f;
    }
  }
}

// The query operand of one pass, in registers: the fp8 limb operand of every
// (pair, MFMA step), the accumulator start (-C_c), the limb weights 32^(4-c)
// of this lane's accumulator rows, and 2^-F times the estimator constant.
template <int T, int QP>
struct QueryOperands {
  static constexpr int IMAGE_BYTES = QP * T * 64 * 32;  // LDS image the operands are built in
  v8i_t A[QP][T];
  v4f_t cinit[QP];
  float wgt[4];
  float qscale[QP];
};

// Build the query operands from the values (all waves of the workgroup take
// part and meet at one LDS barrier).  The caller makes sure no wave still
// reads a previous image.
template <int T, int QP>
__device__ __forceinline__ void build_query_operands(const float (&sv)[2 * QP][2 * T], int nqp,
                                                     int wave, int lane,
                                                     unsigned char *sAimg, float cscale,
                                                     QueryOperands<T, QP> &qo) {
  constexpr int NQ = 2 * QP;
  constexpr int JL = 2 * T;  // m / 64
  const int gq = lane >> 4;
  // ---- per query: exponent F, fixed-point values X_j = rint(Sq_j 2^F),
  // balanced base-32 digits, digit sums C_c (every wave computes these for
  // the whole query) and the operand image (each wave writes the bytes of
  // coordinate blocks j / 64 = wave mod 4).  A query slot past nqp only
  // zeroes its bytes.
  int Fq[NQ];
  int Cq[NQ][5];
#pragma unroll
  for (int qi = 0; qi < NQ; ++qi) {
    Fq[qi] = 0;
#pragma unroll
    for (int c = 0; c < 5; ++c) Cq[qi][c] = 0;
    if (qi >= nqp) {  // empty slot: zero bytes at this wave's coordinates
#pragma unroll
      for (int b = 0; b < JL; ++b) {
        if ((b & 3) != (wave & 3)) continue;
        const int j = lane + 64 * b;
        const int wi = j >> 5, jj = j & 31, sreg = jj & 3;
        const int k = 32 * (wi / T) + 8 * sreg + (jj >> 2);
        const int grp = (k & 63) >> 4, e = (k >> 6) * 16 + (k & 15);
        const uint32_t dst = lds_address(
            sAimg + (((qi >> 1) * T + wi % T) * 64 + 16 * grp + 8 * (qi & 1)) * 32 + e);
        asm volatile(
            "ds_write_b8 %0, %1\n\tds_write_b8 %0, %1 offset:32\n\t"
            "ds_write_b8 %0, %1 offset:64\n\tds_write_b8 %0, %1 offset:96\n\t"
            "ds_write_b8 %0, %1 offset:128\n\tds_write_b8 %0, %1 offset:160\n\t"
            "ds_write_b8 %0, %1 offset:192\n\tds_write_b8 %0, %1 offset:224"
            :
            : "v"(dst), "v"(0u)
            : "memory");
      }
      continue;
    }
    float amax = 0.f;
#pragma unroll
    for (int b = 0; b < JL; ++b) amax = fmaxf(amax, fabsf(sv[qi][b]));
    amax = wave_max_nonneg(amax);
    int e2 = 0;
    (void)frexpf(amax, &e2);
    const int F = amax > 0.f ? 23 - e2 : 0;
    const int qp = qi >> 1, qq = qi & 1;
    int C[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < JL; ++b) {
      const int j = lane + 64 * b;
      const int X = (int)rintf(ldexpf(sv[qi][b], F));
      int L[5];
      int rem = X;
#pragma unroll
      for (int c = 4; c >= 0; --c) {
        L[c] = ((rem + 16) & 31) - 16;
        rem = (rem - L[c]) >> 5;
      }
      // coordinate j -> (MFMA t, lane group, byte e) of the fp8 operand:
      // word wi = j / 32 is fp4 register sreg = j % 4, element eb of lane
      // group gb = wi / T in MFMA t = wi % T; contraction index
      // k = 32 gb + eb sits in fp8 byte e of lane group (k % 64) / 16.
      const int wi = j >> 5, jj = j & 31, sreg = jj & 3;
      const int wj = sreg == 0 ? 5 : (sreg == 3 ? 0 : 1);
#pragma unroll
      for (int c = 0; c < 5; ++c) C[c] += wj * L[c];
      if ((b & 3) == (wave & 3)) {
        const int eb = 8 * sreg + (jj >> 2);
        const int k = 32 * (wi / T) + eb;
        const int t = wi % T;
        const int grp = (k & 63) >> 4, e = (k >> 6) * 16 + (k & 15);
        const int f = sreg == 0 ? 4 : (sreg == 1 ? 2 : (sreg == 2 ? 1 : -1));
        const uint32_t dst =
            lds_address(sAimg + ((qp * T + t) * 64 + 16 * grp + 8 * qq) * 32 + e);
        // Limb rows c = 0..4, zero rows 5..7.  Written in asm: as plain
        // stores the compiler would first wait for any key DMA in flight.
        asm volatile(
            "ds_write_b8 %0, %1\n\tds_write_b8 %0, %2 offset:32\n\t"
            "ds_write_b8 %0, %3 offset:64\n\tds_write_b8 %0, %4 offset:96\n\t"
            "ds_write_b8 %0, %5 offset:128\n\tds_write_b8 %0, %6 offset:160\n\t"
            "ds_write_b8 %0, %6 offset:192\n\tds_write_b8 %0, %6 offset:224"
            :
            : "v"(dst), "v"(e4m3_of_int(f * L[0])), "v"(e4m3_of_int(f * L[1])),
              "v"(e4m3_of_int(f * L[2])), "v"(e4m3_of_int(f * L[3])),
              "v"(e4m3_of_int(f * L[4])), "v"(0u)
            : "memory");
      }
    }
    Fq[qi] = F;
#pragma unroll
    for (int c = 0; c < 5; ++c) Cq[qi][c] = wave_sum(C[c]);
  }
  lds_barrier();  // the image is complete
  // The reads wait for themselves, not for key loads in flight.
#pragma unroll
  for (int qp = 0; qp < QP; ++qp)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      u32x4_t a0, a1;
      asm volatile(
          "ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
          : "=&v"(a0), "=&v"(a1)
          : "v"(lds_address(sAimg + ((qp * T + t) * 64 + lane) * 32))
          : "memory");
      qo.A[qp][t] = v8i_t{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                          (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
  // per-lane epilogue constants: accumulator rows 4 gq + v hold limb
  // c = (4 gq + v) % 8 of query member gq / 2
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = (4 * gq + v) & 7;
    qo.wgt[v] = c < 5 ? (float)(1 << (5 * (4 - c))) : 0.f;
  }
#pragma unroll
  for (int qp = 0; qp < QP; ++qp) {
    const bool hi = (gq >> 1) != 0;
    const int qi0 = 2 * qp, qi1 = 2 * qp + 1;
    const bool qv = (hi ? qi1 : qi0) < nqp;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // limb c = v in even lane groups, c = 4 + v (a limb only for v = 0) in odd ones
      const int lo = hi ? Cq[qi1][v] : Cq[qi0][v];
      const int up = v == 0 ? (hi ? Cq[qi1][4] : Cq[qi0][4]) : 0;
      qo.cinit[qp][v] = qv ? -(float)((gq & 1) ? up : lo) : 0.f;
    }
    const int F = hi ? Fq[qi1] : Fq[qi0];
    qo.qscale[qp] = qv ? ldexpf(cscale, -F) : 0.f;
  }
}

// (m & w) | (~m & c) in one v_bfi_b32 (the compiler emits an AND and an OR
// for a constant c): the mask comes from a scalar register, c from a vector
// register, within the one scalar operand a VOP3 instruction may read.
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t w, uint32_t c) {
  uint32_t d;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(m), "v"(w), "v"(c));
  return d;
}

// One 16-key tile on the matrix cores: expand the bits to the fp4 operand
// and run the MFMAs against the query limbs.  acc[qp] holds the limb rows
// R_c of query pair qp (rows of member 2 qp in lane groups 0-1, of 2 qp + 1
// in lane groups 2-3) for key lane % 16.
template <int T, int QP>
__device__ __forceinline__ void tile_limb_acc(const uint32_t *wb, const QueryOperands<T, QP> &qo,
                                              v4f_t (&acc)[QP]) {
#pragma unroll
  for (int qp = 0; qp < QP; ++qp) acc[qp] = qo.cinit[qp];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint32_t w = wb[t];
    const v8i_t B = v8i_t{(int)bfi(0x11111111u, w, 0x22222222u), (int)(w & 0x22222222u),
                          (int)(w & 0x44444444u), (int)bfi(0x88888888u, w, 0x22222222u),
                          0, 0, 0, 0};
#pragma unroll
    for (int qp = 0; qp < QP; ++qp)
      acc[qp] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.A[qp][t], B, acc[qp], 0, 4,
                                                                  0, 127, 0, 127);
  }
}

// Combine the limb rows a lane holds with those of lane group g ^ 1 (the
// same key, the query's other rows): v_permlane16_swap of a value with
// itself leaves rows (0, 0, 2, 2) in one result and (1, 1, 3, 3) in the
// other, so their sum is v + v[lane ^ 16] with no LDS traffic.  Each limb
// row R_c is an exact integer; their weighted sum sum_c 32^(4-c) R_c =
// sum_j (2 b_j - 1) X_j reaches m 2^23 in magnitude, so the float32 chain
// that forms it rounds, by at most about 2^-24 m max_j |X_j| in all (far
// below the score tolerance once scaled by 2^-F).
__device__ __forceinline__ float limb_rows_combine(const v4f_t &acc, const float (&wgt)[4]) {
  float v = acc[0] * wgt[0];
  v = fmaf(acc[1], wgt[1], v);
  v = fmaf(acc[2], wgt[2], v);
  v = fmaf(acc[3], wgt[3], v);
  const uint32_t x = __float_as_uint(v);
  const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// One 16-key tile: e[qp] is sum_j (2 b_j - 1) X_j of query 2 qp + (lane
// group / 2) against key lane % 16 (in lane groups 0-1 and 2-3 alike): exact
// limb rows, combined in float32 as limb_rows_combine describes.
template <int T, int QP>
__device__ __forceinline__ void tile_limb_sums(const uint32_t *wb, const QueryOperands<T, QP> &qo,
                                               float (&e)[QP]) {
  v4f_t acc[QP];
  tile_limb_acc<T, QP>(wb, qo, acc);
#pragma unroll
  for (int qp = 0; qp < QP; ++qp) e[qp] = limb_rows_combine(acc[qp], qo.wgt);
}

}  // namespace sc
}  // namespace qjl
