// Fused decode attention for several queries per group (grouped-query
// attention): up to four query pairs per pass, with the weighted sum of the
// value rows on the matrix cores.
//
// The step is the one of k_attention.hip (QJL abstract on Majid Daliri's
// scholarfeed page: the sketched keys serve attention; KIVI abstract on the
// same site: a decoding step reads the whole cache):
//     out[g][i][:] = sum_t softmax_t(scale * s[g][i][t]) * V[g][t][:].
// With many queries per pass the per-query weighted sums dominate the vector
// ALUs, so here they become a matrix product per 32-key stage,
//     O[q][d] += sum_t P[q][t] V[t][d],
// on v_mfma_f32_16x16x32_bf16 (queries x dims, 32 keys deep).  The weights P
// are in [0, 1] and are split into three bf16 parts, P = P_hi + P_mid + P_lo
// (24 significant bits, the precision of float32), each multiplied exactly by
// the bf16 values and summed in float32.
//
// Data path per wave, all through a per-wave LDS ring filled by DMA
// (buffer_load ... lds, so no registers are held by loads in flight): per
// 32-key stage the keys' bits and norms, and the 8 KB of value rows.  The
// MFMA B operand needs each lane to hold 8 consecutive keys of one value
// dimension; ds_read_b64_tr_b16 reads them transposed out of the row-major
// rows (measured lane mapping: in each group of 16 lanes, result lane 4x + y
// gets element y of the 8-byte chunks addressed by lanes x, x + 4, x + 8 and
// x + 12).  To keep those reads free of bank conflicts the 8-byte chunk c of
// key k is stored at chunk c ^ 4 g(k), g(k) = (k & 3) | ((k >> 3) & 1) << 2,
// realized by permuting the DMA's source addresses within each row (the DMA
// writes each 1 KB contiguously), so the global reads stay coalesced.
//
// Scores per 16-key tile come from the score kernel's exact fp8-limb MFMA
// sum (score_common.h); the online softmax (maximum and sum per query, exp2
// domain) runs on the vector ALUs; the weights go through a small LDS tile
// (queries x 32 keys, row stride 80 bytes: conflict free) into the MFMA A
// operand.  The four waves merge their states through LDS into one partial
// per query and workgroup, and attn_combine_kernel merges the partials.
#include "attn_common.h"

namespace qjl {

namespace {

using namespace sc;
using namespace at;

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

constexpr int MQ_KEYS = 32;                   // keys per stage (one MFMA contraction)
constexpr int MQ_VBYTES = MQ_KEYS * 2 * AT_DV;  // value rows of a stage: 8 KB
constexpr int MQ_PROW = 80;                   // bytes per query row of the weight tile
constexpr int MQ_PPART = 16 * MQ_PROW;        // one bf16 part: 16 query rows

template <int T>
struct MqRing {
  static constexpr int R = T <= 2 ? 3 : 2;                 // stages in flight per wave
  static constexpr int BITS = MQ_KEYS * 16 * T;            // 512 T bytes
  static constexpr int NORM = 256;                         // 64 lanes x 4 bytes, 32 used
  static constexpr int STAGE = BITS + NORM + MQ_VBYTES;
  static constexpr int NBITS = T >= 2 ? T / 2 : 2;         // bit DMAs: 1 KB each, or 256 B
  static constexpr int L = NBITS + 1 + MQ_VBYTES / 1024;   // DMA instructions per stage
};

// Chunk swizzle of a key row (units of 8 bytes): key k's chunk c sits at
// chunk c ^ mq_swz(k).
__device__ __forceinline__ int mq_swz(int k) {
  return 4 * ((k & 3) | (((k >> 3) & 1) << 2));
}

struct MqSrc {
  __amdgpu_buffer_rsrc_t bits, norm, v;
};

template <int T>
__device__ __forceinline__ MqSrc mq_src(const uint32_t *gbits, const float *gnorm,
                                        const uint16_t *gV, int kbeg, int kend) {
  const uint32_t n = kend > kbeg ? (uint32_t)(kend - kbeg) : 0u;
  return MqSrc{__builtin_amdgcn_make_buffer_rsrc(
                   const_cast<uint32_t *>(gbits + (int64_t)kbeg * 4 * T), (short)0,
                   (int)(n * 16u * T), 0x00020000),
               __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(gnorm + kbeg), (short)0,
                                                 (int)(n * 4u), 0x00020000),
               __builtin_amdgcn_make_buffer_rsrc(
                   const_cast<uint16_t *>(gV + (int64_t)kbeg * AT_DV), (short)0,
                   (int)(n * 2u * AT_DV), 0x00020000)};
}

// DMA of stage keys [k0, k0 + 32) of the workgroup (k0 relative to its first
// key; keys past its end arrive as zeros and are never used).
template <int T>
__device__ __forceinline__ void mq_issue(unsigned char *slot, const MqSrc &src, uint32_t k0,
                                         int lane) {
  typedef __attribute__((address_space(3))) void lds_t;
  if constexpr (T >= 2) {
#pragma unroll
    for (int i = 0; i < T / 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.bits, (lds_t *)(slot + 1024 * i), 16,
                                               (int)(k0 * 16u * T + 1024u * i + 16u * lane), 0,
                                               0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src.bits, (lds_t *)(slot + 256 * i), 4,
                                               (int)(k0 * 16u + 256u * i + 4u * lane), 0, 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.norm, (lds_t *)(slot + MqRing<T>::BITS), 4,
                                           (int)((k0 + lane) * 4u), 0, 0, 0);
  // value rows: DMA j lands keys 4 j .. 4 j + 3 of the stage; lane l fills the
  // 16 bytes at chunk pair l % 16 of key 4 j + l / 16 with the pair that the
  // swizzle puts there
  const int kk0 = lane >> 4, cpl = lane & 15;
#pragma unroll
  for (int j = 0; j < MQ_VBYTES / 1024; ++j) {
    const int kk = 4 * j + kk0;
    const int cp = cpl ^ (mq_swz(kk) >> 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        src.v, (lds_t *)(slot + MqRing<T>::BITS + MqRing<T>::NORM + 1024 * j), 16,
        (int)((k0 + kk) * (2u * AT_DV) + 16u * cp), 0, 0, 0);
  }
}

template <int T>
__device__ __forceinline__ void mq_wait(int pending) {
  constexpr int L = MqRing<T>::L;
  switch (pending) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<L>(); break;
    default: if constexpr (MqRing<T>::R > 2) wait_vmcnt<2 * L>(); break;
  }
}

// The bits of key 16 u + (lane % 16), lane group lane / 16, for the two
// tiles, and the norms of those keys; inline-asm reads that wait for
// themselves (the ring is written by DMA, which the compiler would otherwise
// guard with a full vmcnt(0) before every LDS read).
template <int T>
__device__ __forceinline__ void mq_read_keys(const unsigned char *slot, int lane,
                                             uint32_t (&w)[2][T], float (&n)[2]) {
  const int r = lane & 15, g = lane >> 4;
  const uint32_t a0 = lds_address(slot + r * 16 * T + 4 * T * g);
  const uint32_t an = lds_address(slot + MqRing<T>::BITS + 4 * r);
  if constexpr (T == 1) {
    asm volatile(
        "ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:256\n\t"
        "ds_read_b32 %2, %5\n\tds_read_b32 %3, %5 offset:64\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[1][0]), "=&v"(n[0]), "=&v"(n[1])
        : "v"(a0), "v"(an));
  } else if constexpr (T == 2) {
    u32x2_t x0, x1;
    asm volatile(
        "ds_read_b64 %0, %4\n\tds_read_b64 %1, %4 offset:512\n\t"
        "ds_read_b32 %2, %5\n\tds_read_b32 %3, %5 offset:64\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(n[0]), "=&v"(n[1])
        : "v"(a0), "v"(an));
    w[0][0] = x0.x; w[0][1] = x0.y; w[1][0] = x1.x; w[1][1] = x1.y;
  } else {
    u32x4_t x0, x1;
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b32 %2, %5\n\tds_read_b32 %3, %5 offset:64\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(n[0]), "=&v"(n[1])
        : "v"(a0), "v"(an));
    w[0][0] = x0.x; w[0][1] = x0.y; w[0][2] = x0.z; w[0][3] = x0.w;
    w[1][0] = x1.x; w[1][1] = x1.y; w[1][2] = x1.z; w[1][3] = x1.w;
  }
}

// The MFMA B operands of the stage's value rows: for dim block b (dims
// 16 b .. 16 b + 15), lane l holds dims 16 b + l % 16 of keys 8 (l / 16) ..
// 8 (l / 16) + 7, as two transposed reads of 4 keys each.
__device__ __forceinline__ void mq_read_values(const unsigned char *vbase, int lane,
                                               v8bf_t (&B)[8]) {
  const int s = lane & 15, G = lane >> 4, x = s & 3;
  u32x2_t lo[8], hi[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kk = 8 * G + 4 * h + (s >> 2);
    const int f = mq_swz(kk) >> 2;  // swizzle in units of 32-byte dim blocks
    uint32_t a[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) a[b] = lds_address(vbase + kk * 256 + 32 * (b ^ f) + 8 * x);
    u32x2_t *r = h ? hi : lo;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]));
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v q = {lo[b].x, lo[b].y, hi[b].x, hi[b].y};
    B[b] = __builtin_bit_cast(v8bf_t, q);
  }
}

// bf16 bits of v rounded to nearest even (v finite and >= 0 here).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ws layout: [G * nq][P][AT_PART], one partial per workgroup along the keys
// (P = gridDim.x).  QP query pairs per pass (NQ = 2 QP <= 8 queries: rows of
// the 16-row MFMA past NQ stay zero).
template <int T, int QP>
__global__ __launch_bounds__(SM_THREADS, 1) void attn_mq_kernel(
    const float *__restrict__ Sq, const uint32_t *__restrict__ bits,
    const float *__restrict__ norms, const uint16_t *__restrict__ V, int64_t G, int64_t nq,
    int64_t nk, int chunk, float cscale, float sl2, float *__restrict__ ws,
    float *__restrict__ out) {
  constexpr int W = 4 * T;
  constexpr int m = 32 * W;
  constexpr int NQ = 2 * QP;
  constexpr int JL = m / 64;
  constexpr int R = MqRing<T>::R;
  constexpr int SB = MqRing<T>::STAGE;
  static_assert(NQ <= 8, "two row groups of the MFMA output hold the queries");
  __shared__ __attribute__((aligned(16))) unsigned char sAimg[QueryOperands<T, QP>::IMAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sRing[SM_WAVES][R][SB];
  __shared__ __attribute__((aligned(16))) unsigned char sP[SM_WAVES][3 * MQ_PPART];
  __shared__ __attribute__((aligned(16))) float sPart[SM_WAVES][NQ][AT_PART];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4;
  const int r16 = lane & 15;
  const int P = gridDim.x;
  const int kbeg = (int)blockIdx.x * chunk;
  const int kend = (int64_t)kbeg + chunk < nk ? kbeg + chunk : (int)nk;
  const int nkb = kend > kbeg ? kend - kbeg : 0;
  const int nstage_blk = (nkb + MQ_KEYS - 1) / MQ_KEYS;
  const int ns = (nstage_blk - wave + SM_WAVES - 1) / SM_WAVES;  // this wave's stages

  // rows NQ..15 of the weight tile stay zero (plain stores: nothing is in
  // flight yet)
  for (int i = lane; i < 3 * MQ_PPART / 4; i += 64)
    reinterpret_cast<uint32_t *>(sP[wave])[i] = 0u;

  for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
    const MqSrc src = mq_src<T>(bits + g * nk * (int64_t)W, norms + g * nk,
                                V + g * nk * (int64_t)AT_DV, kbeg, kend);
    for (int64_t q0 = 0; q0 < nq; q0 += NQ) {
      const int nqp = (int)((nq - q0) < NQ ? (nq - q0) : NQ);
      float sv[NQ][JL];
      load_query_values<m, NQ>(Sq + (g * nq + q0) * (int64_t)m, nqp, lane, sv);
#pragma unroll
      for (int j = 0; j < R - 1; ++j)
        mq_issue<T>(&sRing[wave][j][0], src, MQ_KEYS * (wave + SM_WAVES * j), lane);
      wait_vmcnt<(R - 1) * MqRing<T>::L>();  // the query loads, not the stages
      QueryOperands<T, QP> qo;
      build_query_operands<T, QP>(sv, nqp, wave, lane, sAimg, cscale, qo);

      float M[NQ], Lsum[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        M[q] = -INFINITY;
        Lsum[q] = 0.f;
      }
      v4f_t O[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) O[b] = v4f_t{0.f, 0.f, 0.f, 0.f};

      for (int j = 0; j < ns; ++j) {
        mq_issue<T>(&sRing[wave][(j + R - 1) % R][0], src,
                    MQ_KEYS * (wave + SM_WAVES * (j + R - 1)), lane);
        mq_wait<T>(R - 1);
        const unsigned char *slot = &sRing[wave][j % R][0];
        const int k0 = MQ_KEYS * (wave + SM_WAVES * j);
        uint32_t w[2][T];
        float nrm[2];
        mq_read_keys<T>(slot, lane, w, nrm);
        // ---- scores and the online softmax of the stage's 32 keys
        float e[2][QP];
#pragma unroll
        for (int u = 0; u < 2; ++u) tile_limb_sums<T, QP>(w[u], qo, e[u]);
        float p[2][QP];
        float alpha[NQ];
#pragma unroll
        for (int qp = 0; qp < QP; ++qp) {
          const int qi = 2 * qp + (gq >> 1);
          float x[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int key = k0 + 16 * u + r16;
            x[u] = (key < nkb && qi < nqp) ? (e[u][qp] * qo.qscale[qp]) * nrm[u] * sl2
                                           : -INFINITY;
          }
          const float rm = fmaxf(row16_max(x[0]), row16_max(x[1]));
          const float tA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rm), 0));
          const float tB = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rm), 32));
          const float nA = fmaxf(M[2 * qp], tA), nB = fmaxf(M[2 * qp + 1], tB);
          const float mm = (gq >> 1) ? nB : nA;
          p[0][qp] = exp2_shift(x[0], mm);
          p[1][qp] = exp2_shift(x[1], mm);
          const float rs = row16_sum(p[0][qp] + p[1][qp]);
          const float sA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 0));
          const float sB = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 32));
          alpha[2 * qp] = exp2_shift(M[2 * qp], nA);
          alpha[2 * qp + 1] = exp2_shift(M[2 * qp + 1], nB);
          Lsum[2 * qp] = Lsum[2 * qp] * alpha[2 * qp] + sA;
          Lsum[2 * qp + 1] = Lsum[2 * qp + 1] * alpha[2 * qp + 1] + sB;
          M[2 * qp] = nA;
          M[2 * qp + 1] = nB;
        }
        // ---- the weights, three bf16 parts, into the tile [part][query][key]
        {
          unsigned char *pb = sP[wave];
#pragma unroll
          for (int qp = 0; qp < QP; ++qp) {
            const int q = 2 * qp + (gq >> 1);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float v = p[u][qp];
              const uint32_t h0 = bf16_rne(v);
              const float r1 = v - __uint_as_float(h0 << 16);
              const uint32_t s1 = __float_as_uint(r1) >> 31;
              const uint32_t h1 = bf16_rne(fabsf(r1)) | (s1 << 15);
              const float r2 = r1 - __uint_as_float(h1 << 16);
              const uint32_t s2 = __float_as_uint(r2) >> 31;
              const uint32_t h2 = bf16_rne(fabsf(r2)) | (s2 << 15);
              const uint32_t a = lds_address(pb + q * MQ_PROW + 2 * (16 * u + r16));
              asm volatile(
                  "ds_write_b16 %0, %1\n\tds_write_b16 %0, %2 offset:1280\n\t"
                  "ds_write_b16 %0, %3 offset:2560"
                  :
                  : "v"(a), "v"(h0), "v"(h1), "v"(h2));
            }
          }
        }
        // ---- rescale the running sums where a maximum moved
        bool moved = false;
#pragma unroll
        for (int q = 0; q < NQ; ++q) moved |= q < nqp && alpha[q] != 1.f;
        if (moved) {  // uniform
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // output rows of this lane: queries 4 gq + v (rows past NQ unused)
            const float a0 = alpha[v < NQ ? v : 0];
            const float a1 = alpha[4 + v < NQ ? 4 + v : 0];
            const float a = gq == 0 ? a0 : (gq == 1 ? a1 : 1.f);
#pragma unroll
            for (int b = 0; b < 8; ++b) O[b][v] *= a;
          }
        }
        // ---- O += P V on the matrix cores
        v8bf_t Bv[8];
        mq_read_values(slot + MqRing<T>::BITS + MqRing<T>::NORM, lane, Bv);
        u32x4_t ap[3];
        {
          const uint32_t a = lds_address(sP[wave] + r16 * MQ_PROW + 16 * gq);
          asm volatile(
              "ds_read_b128 %0, %3\n\tds_read_b128 %1, %3 offset:1280\n\t"
              "ds_read_b128 %2, %3 offset:2560\n\ts_waitcnt lgkmcnt(0)"
              : "=&v"(ap[0]), "=&v"(ap[1]), "=&v"(ap[2])
              : "v"(a));
        }
#pragma unroll
        for (int part = 0; part < 3; ++part) {
          const v8bf_t A = __builtin_bit_cast(v8bf_t, ap[part]);
#pragma unroll
          for (int b = 0; b < 8; ++b)
            O[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bv[b], O[b], 0, 0, 0);
        }
      }
      wait_vmcnt<0>();  // the ring stages issued past the end
      // ---- this wave's state into LDS: lane l holds rows 4 gq + v, dims
      // 16 b + l % 16
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int q = 4 * gq + v;
        if (q < NQ && q < nqp) {
#pragma unroll
          for (int b = 0; b < 8; ++b) sPart[wave][q][16 * b + r16] = O[b][v];
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          sPart[wave][q][AT_DV] = M[q];
          sPart[wave][q][AT_DV + 1] = Lsum[q];
        }
      }
      __syncthreads();
      // ---- the workgroup's partial of queries wave and wave + 4
#pragma unroll
      for (int hq = 0; hq < 2; ++hq) {
        const int q = wave + SM_WAVES * hq;
        if (q < NQ && q < nqp) {
          float Mw[SM_WAVES], Mx = -INFINITY;
#pragma unroll
          for (int w2 = 0; w2 < SM_WAVES; ++w2) {
            Mw[w2] = sPart[w2][q][AT_DV];
            Mx = fmaxf(Mx, Mw[w2]);
          }
          float Ls = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < SM_WAVES; ++w2) {
            const float f = exp2_shift(Mw[w2], Mx);
            Ls = fmaf(f, sPart[w2][q][AT_DV + 1], Ls);
            o0 = fmaf(f, sPart[w2][q][lane], o0);
            o1 = fmaf(f, sPart[w2][q][lane + 64], o1);
          }
          if (P == 1) {
            // the group's only workgroup: its merged state is the result
            const float inv = 1.f / Ls;
            float *o = out + (g * nq + q0 + q) * (int64_t)AT_DV;
            o[lane] = o0 * inv;
            o[lane + 64] = o1 * inv;
          } else {
            float *dst = ws + ((g * nq + q0 + q) * (int64_t)P + blockIdx.x) * AT_PART;
            dst[lane] = o0;
            dst[lane + 64] = o1;
            if (lane == 0) {
              dst[AT_DV] = Mx;
              dst[AT_DV + 1] = Ls;
            }
          }
        }
      }
      __syncthreads();  // sPart and the query image are free again
    }
  }
}

template <int T, int QP>
void mq_grid(int64_t G, int64_t nk, int64_t *chunk_out, int *gx_out) {
  static PerDevice pd_res;
  const int resident =
      per_device(pd_res, [] { return resident_workgroups(attn_mq_kernel<T, QP>, SM_THREADS); });
  int64_t chunk = (G * nk + resident - 1) / resident;
  constexpr int round = MQ_KEYS * SM_WAVES;
  chunk = (chunk + round - 1) / round * round;
  *chunk_out = chunk;
  *gx_out = (int)((nk + chunk - 1) / chunk);
}

template <int T, int QP>
hipError_t launch_mq_t(const float *Sq, const uint32_t *bits, const float *norms,
                       const uint16_t *V, int64_t G, int64_t nq, int64_t nk, float c, float sl2,
                       float *ws, float *out, int *P_out, hipStream_t st) {
  int64_t chunk = 0;
  int gx = 0;
  mq_grid<T, QP>(G, nk, &chunk, &gx);
  *P_out = gx;
  dim3 grid((unsigned)gx, (unsigned)(G < 65535 ? G : 65535));
  hipLaunchKernelGGL((attn_mq_kernel<T, QP>), grid, dim3(SM_THREADS), 0, st, Sq, bits, norms, V,
                     G, nq, nk, (int)chunk, c, sl2, ws, out);
  return hipGetLastError();
}

template <int T>
hipError_t launch_mq_qp(const float *Sq, const uint32_t *bits, const float *norms,
                        const uint16_t *V, int64_t G, int64_t nq, int64_t nk, float c, float sl2,
                        float *ws, float *out, int *P_out, hipStream_t st) {
  // eight queries per pass once there are more than four
  if (nq > 4) return launch_mq_t<T, 4>(Sq, bits, norms, V, G, nq, nk, c, sl2, ws, out, P_out, st);
  return launch_mq_t<T, 2>(Sq, bits, norms, V, G, nq, nk, c, sl2, ws, out, P_out, st);
}

template <int T>
int mq_partials_t(int64_t G, int64_t nk) {
  int64_t chunk = 0;
  int gx2 = 0, gx4 = 0;
  mq_grid<T, 2>(G, nk, &chunk, &gx2);
  mq_grid<T, 4>(G, nk, &chunk, &gx4);
  return gx2 > gx4 ? gx2 : gx4;
}

}  // namespace

bool attn_mq_supported(int T) { return T == 1 || T == 2 || T == 4; }

int attn_mq_partials(int T, int64_t G, int64_t nk) {
  switch (T) {
    case 1: return mq_partials_t<1>(G, nk);
    case 2: return mq_partials_t<2>(G, nk);
    case 4: return mq_partials_t<4>(G, nk);
  }
  return 0;
}

hipError_t launch_attn_mq_partials(int T, const float *Sq, const uint32_t *bits,
                                   const float *norms, const uint16_t *V, int64_t G, int64_t nq,
                                   int64_t nk, float c, float sl2, float *ws, float *out,
                                   int *P_out, hipStream_t st) {
  switch (T) {
    case 1: return launch_mq_qp<1>(Sq, bits, norms, V, G, nq, nk, c, sl2, ws, out, P_out, st);
    case 2: return launch_mq_qp<2>(Sq, bits, norms, V, G, nq, nk, c, sl2, ws, out, P_out, st);
    case 4: return launch_mq_qp<4>(Sq, bits, norms, V, G, nq, nk, c, sl2, ws, out, P_out, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qjl
