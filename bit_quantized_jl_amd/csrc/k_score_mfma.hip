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
//     groups 0 and 1, or 2 and 3; v_permlane16_swap adds the two groups),
//     moves the scores of a 64-key stage to one key per lane with
//     v_permlane32_swap, scales by c ||k|| 2^-F and stores them with one
//     non-temporal 256-byte store per query (the scores are not read again
//     by this kernel).
//
// Set-up per workgroup and query pass: each wave loads the query values,
// starts its key stream, then computes F and the digit sums for the whole
// query itself and writes the operand bytes of a quarter of the coordinates
// into one shared LDS image; a single LDS barrier later every wave reads its
// operand registers.  No wave waits for the key stream during the set-up.
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
#include "score_common.h"

namespace qjl {

namespace {

using namespace sc;

typedef __attribute__((address_space(3))) void lds_void_t;

// Keys stream through a per-wave LDS ring filled by buffer_load ... lds (the
// direct HBM -> LDS path): no registers are held by loads in flight,
// so a wave keeps R - 1 stages of 64 keys outstanding while it computes one.
constexpr int SM_STAGE = 64;  // keys per stage (4 MFMA tiles of 16)
// The first R - 1 stages are issued unconditionally (a stage past the
// workgroup's keys reads zeros and is never consumed), so the number of loads
// in flight is static when the loop starts.

template <int T>
struct Ring {
  static constexpr int BITS_BYTES = SM_STAGE * 16 * T;     // 64 keys x 4T words
  static constexpr int STAGE_BYTES = BITS_BYTES + SM_STAGE * 4;
  static constexpr int L = T + 1;                          // DMA instructions per stage
};

// Stages in the ring.  One query pair per pass, from m = 256 up: two (one
// stage in flight while one is computed), which measured faster than three
// or four (7B decode 15.8-15.9 against 16.4-16.6 us with four workgroups per
// group, long context 51.6-51.7 against 53.0-53.1 us).  More query pairs per
// pass compute longer per stage and keep the deeper rings: with two stages,
// eight and sixteen queries per group took 47 and 91 against 41 and 79 us.
template <int T, int QP>
constexpr int ring_depth() {
  if (QP == 1 && T >= 2) return 2;
  return T <= 2 ? 4 : (T <= 4 ? 3 : 2);
}

template <int T, int R>
__device__ __forceinline__ void wait_stages(int pending) {
  constexpr int L = Ring<T>::L;
  switch (pending) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<L>(); break;
    case 2: if constexpr (R > 2) wait_vmcnt<2 * L>(); break;
    default: if constexpr (R > 3) wait_vmcnt<3 * L>(); break;
  }
}

// Buffer descriptors over the workgroup's keys [kbeg, kend) of a group: a
// DMA past kend reads zeros (the descriptor's range check), so no address is
// clamped, and every offset is a 32-bit register.  The keys of one
// workgroup span less than 4 GB (the whole cache fits in HBM and is split
// over hundreds of workgroups).
struct StageSrc {
  __amdgpu_buffer_rsrc_t bits, norm;
};

template <int T>
__device__ __forceinline__ StageSrc stage_src(const uint32_t *gbits, const float *gnorm,
                                              int64_t kbeg, int64_t kend) {
  constexpr int W = 4 * T;
  const uint32_t n = kend > kbeg ? (uint32_t)(kend - kbeg) : 0u;
  return StageSrc{
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(gbits + kbeg * W), (short)0,
                                        (int)(n * (uint32_t)(4 * W)), 0x00020000),
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(gnorm + kbeg), (short)0,
                                        (int)(n * 4u), 0x00020000)};
}

// Issue the DMA of one stage: keys [k0, k0 + 64) of the workgroup (k0
// relative to its first key; keys past its end land as zeros and their
// results are never stored).  The stage's bits are one contiguous run of
// 64 W words, so DMA instruction i moves bytes [1024 i, 1024 i + 1024).
template <int T>
__device__ __forceinline__ void issue_stage(unsigned char *slot, const StageSrc &src, uint32_t k0,
                                            int lane) {
  constexpr int W = 4 * T;
#pragma unroll
  for (int i = 0; i < T; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.bits, (lds_void_t *)(slot + i * 1024), 16,
                                             (int)(k0 * (4u * W) + i * 1024u + lane * 16u), 0, 0,
                                             0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src.norm, (lds_void_t *)(slot + Ring<T>::BITS_BYTES), 4,
                                           (int)((k0 + lane) * 4u), 0, 0, 0);
}

// Read one ring stage for this lane: the T words of key 16 u + (lane % 16),
// lane group lane / 16, for the 4 tiles u, and the norm of key `lane` of the
// stage.  The reads are inline asm that waits for its own results: the ring
// is written by DMA, which the compiler would otherwise guard with a full
// vmcnt(0) before every read (the explicit wait_stages() before this call
// is the real guard).
template <int T>
struct StageRead;

template <>
struct StageRead<1> {
  uint32_t w[4][1];
  float n;
  __device__ __forceinline__ void read(uint32_t aw, uint32_t an) {
    asm volatile(
        "ds_read_b32 %0, %5\n\tds_read_b32 %1, %5 offset:256\n\t"
        "ds_read_b32 %2, %5 offset:512\n\tds_read_b32 %3, %5 offset:768\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[1][0]), "=&v"(w[2][0]), "=&v"(w[3][0]), "=&v"(n)
        : "v"(aw), "v"(an));
  }
};

template <>
struct StageRead<2> {
  uint32_t w[4][2];
  float n;
  __device__ __forceinline__ void read(uint32_t aw, uint32_t an) {
    u32x2_t a, b, c, d;
    asm volatile(
        "ds_read_b64 %0, %5\n\tds_read_b64 %1, %5 offset:512\n\t"
        "ds_read_b64 %2, %5 offset:1024\n\tds_read_b64 %3, %5 offset:1536\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(n)
        : "v"(aw), "v"(an));
    w[0][0] = a.x; w[0][1] = a.y; w[1][0] = b.x; w[1][1] = b.y;
    w[2][0] = c.x; w[2][1] = c.y; w[3][0] = d.x; w[3][1] = d.y;
  }
};

template <>
struct StageRead<4> {
  uint32_t w[4][4];
  float n;
  __device__ __forceinline__ void read(uint32_t aw, uint32_t an) {
    u32x4_t a, b, c, d;
    asm volatile(
        "ds_read_b128 %0, %5\n\tds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b128 %2, %5 offset:2048\n\tds_read_b128 %3, %5 offset:3072\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(n)
        : "v"(aw), "v"(an));
    const u32x4_t v[4] = {a, b, c, d};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u][0] = v[u].x; w[u][1] = v[u].y; w[u][2] = v[u].z; w[u][3] = v[u].w;
    }
  }
};

template <>
struct StageRead<8> {
  uint32_t w[4][8];
  float n;
  __device__ __forceinline__ void read(uint32_t aw, uint32_t an) {
    u32x4_t a0, a1, b0, b1, c0, c1, d0, d1;
    asm volatile(
        "ds_read_b128 %0, %9\n\tds_read_b128 %1, %9 offset:16\n\t"
        "ds_read_b128 %2, %9 offset:2048\n\tds_read_b128 %3, %9 offset:2064\n\t"
        "ds_read_b128 %4, %9 offset:4096\n\tds_read_b128 %5, %9 offset:4112\n\t"
        "ds_read_b128 %6, %9 offset:6144\n\tds_read_b128 %7, %9 offset:6160\n\t"
        "ds_read_b32 %8, %10\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1), "=&v"(c0), "=&v"(c1), "=&v"(d0),
          "=&v"(d1), "=&v"(n)
        : "v"(aw), "v"(an));
    const u32x4_t v[8] = {a0, a1, b0, b1, c0, c1, d0, d1};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u][0] = v[2 * u].x; w[u][1] = v[2 * u].y; w[u][2] = v[2 * u].z; w[u][3] = v[2 * u].w;
      w[u][4] = v[2 * u + 1].x; w[u][5] = v[2 * u + 1].y;
      w[u][6] = v[2 * u + 1].z; w[u][7] = v[2 * u + 1].w;
    }
  }
};

// One 64-key stage: the MFMAs of its four tiles first (independent
// accumulators, so they issue back to back), then the limb combination, then
// the scores move to one key per lane -- lane l gets key l of the stage,
// member A of each query pair in one register and member B in the other --
// by two selects and one v_permlane32_swap (tile u's keys sit in lane group
// u % 2 of select source u / 2), and leave with one 256-byte store per query.
// The query scale lives in the lane groups of its member (A: 0-1, B: 2-3),
// so each member's is read from one of its lanes.
template <int T, int QP, bool DEFER>
__device__ __forceinline__ void score_stage(const StageRead<T> &sr, const QueryOperands<T, QP> &qo,
                                            int64_t key, int64_t kbeg, int64_t kend, int gq,
                                            int nqp, float *__restrict__ outq, int64_t nk,
                                            float *sDefer, int chunk) {
  v4f_t acc[4][QP];
#pragma unroll
  for (int u = 0; u < 4; ++u) tile_limb_acc<T, QP>(sr.w[u], qo, acc[u]);
  const bool odd = gq & 1;
#pragma unroll
  for (int qp = 0; qp < QP; ++qp) {
    float e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = limb_rows_combine(acc[u][qp], qo.wgt);
    const uint32_t x = __float_as_uint(odd ? e[1] : e[0]);
    const uint32_t y = __float_as_uint(odd ? e[3] : e[2]);
    const auto sw = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    const uint32_t qs = __float_as_uint(qo.qscale[qp]);
    const float sa = __uint_as_float(__builtin_amdgcn_readlane(qs, 0)) * sr.n;
    const float sb = __uint_as_float(__builtin_amdgcn_readlane(qs, 32)) * sr.n;
    if (key < kend) {
      const int qa = 2 * qp, qb = 2 * qp + 1;
      if constexpr (DEFER) {
        const int kl = (int)(key - kbeg);
        if (qa < nqp) sDefer[qa * chunk + kl] = __uint_as_float(sw[0]) * sa;
        if (qb < nqp) sDefer[qb * chunk + kl] = __uint_as_float(sw[1]) * sb;
      } else {
        if (qa < nqp) __builtin_nontemporal_store(__uint_as_float(sw[0]) * sa, outq + qa * nk + key);
        if (qb < nqp) __builtin_nontemporal_store(__uint_as_float(sw[1]) * sb, outq + qb * nk + key);
      }
    }
  }
}

// With DEFER the scores of a pass stay in LDS (sDefer: [queries][chunk]) and
// each wave writes those of its own stages as 16-byte non-temporal stores when
// its last stage is done; otherwise each stage stores its own.
template <int T, int QP, bool DEFER>
__global__ __launch_bounds__(SM_THREADS) void score_mfma_kernel(
    const float *__restrict__ Sq, const uint32_t *__restrict__ bits,
    const float *__restrict__ norms, int64_t G, int64_t nq, int64_t nk, int chunk, float cscale,
    float *__restrict__ out) {
  constexpr int W = 4 * T;         // 32-bit words per key (m = 128 T)
  constexpr int m = 32 * W;
  constexpr int NQ = 2 * QP;       // queries per pass
  constexpr int R = ring_depth<T, QP>();
  constexpr int SB = Ring<T>::STAGE_BYTES;
  constexpr int JL = (m + 63) / 64;            // query coordinates per lane
  __shared__ __attribute__((aligned(16))) unsigned char sAimg[QueryOperands<T, QP>::IMAGE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char sRing[SM_WAVES][R][SB];
  extern __shared__ __attribute__((aligned(16))) float sDefer[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int gq = lane >> 4;  // lane group 0..3
  const int64_t kbeg = (int64_t)blockIdx.x * chunk;
  const int64_t kend = (kbeg + chunk) < nk ? (kbeg + chunk) : nk;
  // this wave's stages: kbeg + 64 (wave + 4 j), j < ns
  const int64_t nstage_blk = (kend - kbeg + SM_STAGE - 1) / SM_STAGE;
  const int ns = (int)((nstage_blk - wave + SM_WAVES - 1) / SM_WAVES);

  for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
    const StageSrc src = stage_src<T>(bits + g * nk * (int64_t)W, norms + g * nk, kbeg, kend);
    for (int64_t q0 = 0; q0 < nq; q0 += NQ) {
      const int nqp = (int)((nq - q0) < NQ ? (nq - q0) : NQ);
      // ---- query values first (plain loads), then the first key stages
      // (LDS DMA), so the query set-up below overlaps the stream's latency.
      float sv[NQ][JL];
      load_query_values<m, NQ>(Sq + (g * nq + q0) * (int64_t)m, nqp, lane, sv);
#pragma unroll
      for (int j = 0; j < R - 1; ++j)
        issue_stage<T>(&sRing[wave][j][0], src, SM_STAGE * (wave + SM_WAVES * j), lane);
      // The query loads are the oldest in flight: wait for them alone.  (The
      // compiler cannot count past LDS DMA and would wait for the stages too.)
      wait_vmcnt<(R - 1) * Ring<T>::L>();
      if (q0 > 0) lds_barrier();  // every wave has read the previous pass's image
      QueryOperands<T, QP> qo;
      build_query_operands<T, QP>(sv, nqp, wave, lane, sAimg, cscale, qo);
      // ---- stream this wave's stages through the ring
      for (int j = 0; j < ns; ++j) {
        if (j + R - 1 < ns)
          issue_stage<T>(&sRing[wave][(j + R - 1) % R][0], src,
                         SM_STAGE * (wave + SM_WAVES * (j + R - 1)), lane);
        // stages issued after stage j: up to the last real one, and at least
        // the R - 2 issued before the loop
        const int last = (ns - 1) < (j + R - 1) ? (ns - 1) : (j + R - 1);
        wait_stages<T, R>((last > R - 2 ? last : R - 2) - j);
        const unsigned char *slot = &sRing[wave][j % R][0];
        const int64_t k0 = kbeg + SM_STAGE * (wave + SM_WAVES * j);
        StageRead<T> sr;
        sr.read(lds_address(slot + ((lane & 15) * W + T * gq) * 4),
                lds_address(slot + Ring<T>::BITS_BYTES + lane * 4));
        score_stage<T, QP, DEFER>(sr, qo, k0 + lane, kbeg, kend, gq, nqp,
                                  out + (g * nq + q0) * nk, nk, sDefer, chunk);
      }
      if constexpr (DEFER) {
        // each wave writes the scores of its own 64-key blocks (keys
        // kbeg + 64 (wave + 4 j)) as soon as its stages are done: it wrote
        // those LDS slots itself, so no workgroup barrier is needed; 16 lanes
        // cover one block, four consecutive keys each
        __builtin_amdgcn_s_waitcnt((15 & 15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        const int nkb = (int)(kend - kbeg);
        for (int qi = 0; qi < nqp; ++qi) {
          float *dst = out + (g * nq + q0 + qi) * nk + kbeg;
          const float *srcq = sDefer + qi * chunk;
          const bool vec = ((uintptr_t)dst & 15) == 0;
          for (int j = lane >> 4; j < ns; j += 4) {
            const int i = SM_STAGE * (wave + SM_WAVES * j) + 4 * (lane & 15);
            if (vec && i + 3 < nkb) {
              const v4f_t v = *reinterpret_cast<const v4f_t *>(srcq + i);
              __builtin_nontemporal_store(v, reinterpret_cast<v4f_t *>(dst + i));
            } else {
              for (int t = 0; t < 4 && i + t < nkb; ++t)
                __builtin_nontemporal_store(srcq[i + t], dst + i + t);
            }
          }
        }
        asm volatile("" ::: "memory");
      }
    }
  }
  wait_vmcnt<0>();  // DMA of stages past the end must land before exit
}

// LDS the deferred scores may take per workgroup (beside the ring and the
// query image, within the 160 KB of a compute unit).
constexpr size_t DEFER_MAX_BYTES = 64 << 10;

// The dynamic LDS a deferring launch of score_mfma_kernel<T, QP, true> may
// take on the current device: DEFER_MAX_BYTES, or less where the kernel's
// static LDS leaves less room within a workgroup's limit (m = 1024: the
// stage ring and the query image already take most of it); 0 when the
// kernel's attribute cannot be raised (then the scores are stored per stage).
// The attribute is set once per device; a refusal is cleared from the
// runtime's last-error state so that it does not surface as a launch error.
template <int T, int QP>
size_t defer_limit() {
  static PerDevice pd;
  return (size_t)(per_device(pd, [] {
    int dev = 0, max_block = 0;
    hipFuncAttributes a{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&max_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        hipFuncGetAttributes(&a, (const void *)score_mfma_kernel<T, QP, true>) != hipSuccess) {
      (void)hipGetLastError();
      return 1;
    }
    const int64_t room = (int64_t)max_block - (int64_t)a.sharedSizeBytes;
    const int lim = (int)(room < (int64_t)DEFER_MAX_BYTES ? room : (int64_t)DEFER_MAX_BYTES);
    if (lim <= 0) return 1;
    if (hipFuncSetAttribute((const void *)score_mfma_kernel<T, QP, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lim) != hipSuccess) {
      (void)hipGetLastError();
      return 1;
    }
    return lim + 1;
  }) - 1);
}

template <int T, int QP, bool DEFER>
void launch_sm_kernel(dim3 grid, size_t dyn, hipStream_t st, const float *Sq,
                      const uint32_t *bits, const float *norms, int64_t G, int64_t nq,
                      int64_t nk, int chunk, float c, float *scores) {
  hipLaunchKernelGGL((score_mfma_kernel<T, QP, DEFER>), grid, dim3(SM_THREADS), dyn, st, Sq,
                     bits, norms, G, nq, nk, chunk, c, scores);
}

template <int T, int QP>
hipError_t launch_sm(const float *Sq, const uint32_t *bits, const float *norms, int m, int64_t G,
                     int64_t nq, int64_t nk, float c, float *scores, hipStream_t st) {
  (void)m;
  // One workgroup per compute unit: the keys of all groups in equal chunks
  // (long context: 57.5 against 61.3 us for the resident round of two or
  // three workgroups per unit, which set up each query more often).
  static PerDevice pd_res, pd_cus;
  const int resident =
      per_device(pd_res, [] { return resident_workgroups(score_mfma_kernel<T, QP, false>, SM_THREADS); });
  const int cus = per_device(pd_cus, device_compute_units);
  static PerDevice pd_lds, pd_static;
  const int lds_cu = per_device(pd_lds, [] {
    int dev = 0, v = 0;
    (void)hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess || v <= 0) {
      (void)hipGetLastError();  // a failed query is not a launch error
      v = 160 << 10;
    }
    return v;
  });
  const int lds_static = per_device(pd_static, [] {
    hipFuncAttributes a{};
    if (hipFuncGetAttributes(&a, (const void *)score_mfma_kernel<T, QP, true>) != hipSuccess) {
      (void)hipGetLastError();  // a failed query is not a launch error
      return 1 << 30;           // unknown: never defer
    }
    return (int)a.sharedSizeBytes + 1;
  }) - 1;
  // Scores written per stage cost more than the same bytes written in one
  // burst per workgroup (long context: 56 against 53.5 us): a launch defers
  // them to LDS when a pass's scores of the workgroup's keys fit and the
  // extra LDS leaves as many of its workgroups resident at once.
  const int64_t nqd = nq < 2 * QP ? nq : 2 * QP;
  const int64_t per_cu_plain = resident / cus;
  auto defers = [&](int64_t ch, int64_t wgs) {
    const size_t dyn = (size_t)(nqd * ch) * sizeof(float);
    const int64_t per_cu_defer = (int64_t)lds_cu / ((int64_t)lds_static + (int64_t)dyn);
    const int64_t need_per_cu = (wgs + cus - 1) / cus;
    const int64_t want = need_per_cu < per_cu_plain ? need_per_cu : per_cu_plain;
    return dyn > 0 && dyn <= defer_limit<T, QP>() && per_cu_defer >= want;
  };
  auto chunk_of = [&](int64_t parts) { return ((nk + parts - 1) / parts + 255) / 256 * 256; };
  // chunk: a multiple of the 256 keys one block step covers
  int64_t chunk = (G * nk + cus - 1) / cus;
  chunk = (chunk + 255) / 256 * 256;
  // With a group per compute unit or more, each group splits into equal parts
  // (no short last chunk as in the resident-round split: two halves took 18.0
  // against 19.1 us at the 7B decode shape; one workgroup per group leaves the
  // chip a wave per SIMD and is slower).  Four parts, where all stay resident
  // and still defer their scores: 15.8-15.9 against 16.4-16.6 us for two (17.4
  // us for eight) at the 7B decode shape; with eight or sixteen queries per
  // group, whose scores are stored per stage, four parts were slower (47 and
  // 91 against 41 and 79 us), so those keep two.
  if (G >= cus && 2 * G <= resident) {
    const int64_t c4 = chunk_of(4);
    const int64_t rows = G < 65535 ? G : 65535;  // the grid's groups at a time
    chunk = 4 * G <= resident && defers(c4, rows * ((nk + c4 - 1) / c4)) ? c4 : chunk_of(2);
  }
  dim3 grid((unsigned)((nk + chunk - 1) / chunk), (unsigned)(G < 65535 ? G : 65535));
  const size_t dyn = (size_t)(nqd * chunk) * sizeof(float);
  if (defers(chunk, (int64_t)grid.x * grid.y))
    launch_sm_kernel<T, QP, true>(grid, dyn, st, Sq, bits, norms, G, nq, nk, (int)chunk, c, scores);
  else
    launch_sm_kernel<T, QP, false>(grid, 0, st, Sq, bits, norms, G, nq, nk, (int)chunk, c, scores);
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
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_score(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                        const float *norms, int64_t G, int64_t nq, int64_t nk, float *scores,
                        hipStream_t st) {
  const int m = sk->host.m;
  // the MFMA path covers m = 128 T, T <= 8, with 16-byte aligned bits
  if (m > 1024 || m % 128 != 0 || ((uintptr_t)bits & 15) != 0)
    return launch_score_generic(sk, Sq, bits, norms, G, nq, nk, scores, st);
  const int W = m / 32;
  const int T = W / 4;
  // up to four query pairs per pass (eight pairs measured slower: one
  // workgroup per CU and spills; two passes of four re-read the bits instead)
  const int qp_max = T <= 4 ? 4 : 2;
  int qp = 1;
  while (qp < qp_max && 2 * qp < nq) qp *= 2;
  const float c = estimator_scale(m, sk->host.rho);
  switch (T) {
    case 1: return launch_sm_t<1>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 2: return launch_sm_t<2>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 4: return launch_sm_t<4>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
    case 8: return launch_sm_t<8>(qp, Sq, bits, norms, m, G, nq, nk, c, scores, st);
  }
  return launch_score_generic(sk, Sq, bits, norms, G, nq, nk, scores, st);
}

}  // namespace qjl
