// Fused decode-step attention on the QJL scores.
//
// For query i of group g (QJL abstract on Majid Daliri's scholarfeed page:
// the sketched keys serve attention; the KIVI abstract on the same site: a
// decoding step reads the whole KV cache once):
//     out[g][i][:] = sum_t softmax_t(scale * s[g][i][t]) * V[g][t][:],
// with s the QJL estimate of q.k (the score of k_score_mfma.hip).  The scores
// never reach HBM: each wave scores a 16-key tile on the matrix cores (the
// exact fp8-limb method of the score kernel, shared through score_common.h),
// folds it into an online softmax (running maximum and sum, in the exp2
// domain) and adds the weighted value rows.  The four waves of a workgroup
// merge their states through LDS into one partial (maximum, sum, d_v-float
// weighted sum) per query in the caller's workspace; attn_combine_kernel
// merges the partials of a query.
//
// The stream uses plain loads into registers, a ring of 16-key stages: the
// bits and norms of a stage (as the score kernel loads them) and its value
// rows, lane l holding bf16 dimensions [8 (l % 16), 8 (l % 16) + 8) of key
// 4 j + l / 16 of each 16-key tile (one 16-byte load covers four rows).
// (LDS DMA for the bits, as in the score kernel, would make the compiler wait
// for every load before using the value registers.)
//
// This kernel serves one or two queries per group (and m = 1024); three or
// more take attn_mq_kernel (k_attention_mq.hip), whose weighted sums run on
// the matrix cores.  Shapes neither fast path covers (d_v != 128, float
// values, m other than 128, 256, 512 or 1024, unaligned buffers, 2^22 keys or
// more per group) take a plain path: the score kernel writes the scores to
// the workspace and attn_softmax_kernel forms the weighted sum.
#include "attn_common.h"

namespace qjl {

namespace {

using namespace sc;
using namespace at;

constexpr int AT_TILES = 1;   // 16-key tiles per stage
constexpr int AT_STAGE = 16 * AT_TILES;  // keys per stage

template <int T>
struct AttnStage {
  uint32_t w[AT_TILES][T];  // bits: words [T g, T g + T) of key 16 u + lane % 16
  float n;                  // norm of key lane % 32 of the stage
  uint4 v[AT_TILES][4];     // values: tile u, row 4 j + lane / 16, dims 8 (lane % 16) ..
};

// Buffer descriptors over keys [kbeg, kend) of a group: a load past kend
// returns zeros (the descriptor's range check), so a stage needs no per-lane
// clamps and every address is a 32-bit offset from the descriptor's base.
struct KeyRange {
  __amdgpu_buffer_rsrc_t bits, norm, v;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_rsrc(const void *base, int kbeg, int kend,
                                                           int bytes_per_key) {
  const uint32_t n = kend > kbeg ? (uint32_t)(kend - kbeg) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(static_cast<const char *>(base) + (int64_t)kbeg * bytes_per_key),
      (short)0, (int)(n * (uint32_t)bytes_per_key), 0x00020000);
}

template <int T>
__device__ __forceinline__ KeyRange key_range(const uint32_t *gbits, const float *gnorm,
                                              const uint16_t *gV, int kbeg, int kend) {
  return KeyRange{key_rsrc(gbits, kbeg, kend, 16 * T), key_rsrc(gnorm, kbeg, kend, 4),
                  key_rsrc(gV, kbeg, kend, 2 * AT_DV)};
}

// Stage of keys [k0, k0 + AT_STAGE), k0 relative to the range's first key.
template <int T>
__device__ __forceinline__ void load_attn_stage(AttnStage<T> &s, const KeyRange &kr, int k0,
                                                int lane) {
  constexpr int W = 4 * T;
  const int r = lane & 15, gq = lane >> 4;
#pragma unroll
  for (int u = 0; u < AT_TILES; ++u) {
    const int off = (int)(((uint32_t)(k0 + 16 * u + r) * W + T * gq) * 4u);
    if constexpr (T == 1) {
      s.w[u][0] = __builtin_amdgcn_raw_buffer_load_b32(kr.bits, off, 0, 0);
    } else if constexpr (T == 2) {
      const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(kr.bits, off, 0, 0);
      s.w[u][0] = v.x;
      s.w[u][1] = v.y;
    } else {
#pragma unroll
      for (int h = 0; h < T / 4; ++h) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(kr.bits, off + 16 * h, 0, 0);
        s.w[u][4 * h] = v.x;
        s.w[u][4 * h + 1] = v.y;
        s.w[u][4 * h + 2] = v.z;
        s.w[u][4 * h + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
          kr.v, (int)((uint32_t)(k0 + 16 * u + 4 * j + gq) * (2u * AT_DV) + 16u * r), 0, 0);
      s.v[u][j] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  s.n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
      kr.norm, (int)(4u * (uint32_t)(k0 + (lane & (AT_STAGE - 1)))), 0, 0));
}

// Running softmax state of the queries a lane serves: per query pair qp,
// member A = 2 qp and B = 2 qp + 1; M and L are the same in every lane.
template <int QP>
struct SoftmaxState {
  float M[QP][2], L[QP][2];
  float acc[QP][2][8];
};

// PAIR: both members of the query pair exist (else only member A's weighted
// sum is formed).
template <int T, int QP, bool PAIR>
__device__ __forceinline__ void attn_stage(const AttnStage<T> &s, const QueryOperands<T, QP> &qo,
                                           int k0, int kend, int lane, int nqp,
                                           float sl2, SoftmaxState<QP> &st) {
  const int gq = lane >> 4;
#pragma unroll
  for (int u = 0; u < AT_TILES; ++u) {
    const int key = k0 + 16 * u + (lane & 15);
    float e[QP];
    tile_limb_sums<T, QP>(s.w[u], qo, e);
    const float nrm = __shfl(s.n, 16 * u + (lane & 15));
    float vals[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t q[4] = {s.v[u][j].x, s.v[u][j].y, s.v[u][j].z, s.v[u][j].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        vals[j][2 * h] = __uint_as_float(q[h] << 16);
        vals[j][2 * h + 1] = __uint_as_float(q[h] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int qp = 0; qp < QP; ++qp) {
      if (2 * qp >= nqp) break;  // uniform
      const int qi = 2 * qp + (gq >> 1);
      // logit in the exp2 domain: scale * log2(e) * score
      const float x = (key < kend && qi < nqp) ? (e[qp] * qo.qscale[qp]) * nrm * sl2 : -INFINITY;
      const float rm = row16_max(x);
      const float tA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rm), 0));
      const float tB = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rm), 32));
      const float nA = fmaxf(st.M[qp][0], tA), nB = fmaxf(st.M[qp][1], tB);
      const float p = exp2_shift(x, (gq >> 1) ? nB : nA);
      const float rs = row16_sum(p);
      const float sA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 0));
      const float sB = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs), 32));
      const float aA = exp2_shift(st.M[qp][0], nA), aB = exp2_shift(st.M[qp][1], nB);
      st.L[qp][0] = st.L[qp][0] * aA + sA;
      st.L[qp][1] = st.L[qp][1] * aB + sB;
      st.M[qp][0] = nA;
      st.M[qp][1] = nB;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        st.acc[qp][0][d] *= aA;
        if (PAIR) st.acc[qp][1][d] *= aB;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + gq;  // key of this lane's value row in the tile
        const float pA = __shfl(p, t);
        const float pB = PAIR ? __shfl(p, 32 + t) : 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          st.acc[qp][0][d] = fmaf(pA, vals[j][d], st.acc[qp][0][d]);
          if (PAIR) st.acc[qp][1][d] = fmaf(pB, vals[j][d], st.acc[qp][1][d]);
        }
      }
      if (QP > 1) __builtin_amdgcn_sched_barrier(0);  // one pair's temporaries at a time
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Stages held in registers per wave: one is computed while the others load.
// Three, except two for a single query from m = 512 up: at long context
// (m = 512) one query took 219.9 against 226.4 us with three, but a query
// pair 239.4 against 221.3 us; at the 7B decode shape (m = 256) three stay
// faster for one query too (101.8 against 105.1 us with two).
template <int T, bool PAIR>
constexpr int attn_ring() {
  return T >= 4 && !PAIR ? 2 : 3;
}

// The key stream of one wave: the workgroup's stages wave, wave + 4, ...
// (stage i: keys key0 + kstride i + [0, AT_STAGE) of the range) through a
// ring of R register stages (stage i lives in b[i % R]).
template <int T, int QP, bool PAIR, int R>
__device__ __forceinline__ void stream_keys(AttnStage<T> (&b)[R], const KeyRange &kr,
                                            const QueryOperands<T, QP> &qo, int wave, int lane,
                                            int nsr, int key0, int kstride, int nkb, int nqp,
                                            float sl2, SoftmaxState<QP> &st) {
  for (int j = 0; j < nsr; j += R) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k0 = key0 + kstride * (wave + SM_WAVES * (j + r));
      attn_stage<T, QP, PAIR>(b[r], qo, k0, nkb, lane, nqp, sl2, st);
      load_attn_stage<T>(b[r], kr, k0 + kstride * R * SM_WAVES, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ws layout: [G * nq][P][AT_PART], one partial per workgroup along the keys
// (P = gridDim.x): the weighted sum, then M and L (exp2 domain).  A pass
// serves QP query pairs (QP <= 2: one merging wave per query); PAIR is
// nq > 1 (with one query per group, member B's sums are never formed).
template <int T, int QP, bool PAIR>
__global__ __launch_bounds__(SM_THREADS, QP == 1 ? 2 : 1) void attn_partial_kernel(
    const float *__restrict__ Sq, const uint32_t *__restrict__ bits,
    const float *__restrict__ norms, const uint16_t *__restrict__ V, int64_t G, int64_t nq,
    int64_t nk, int chunk, int inter, float cscale, float sl2, float *__restrict__ ws,
    float *__restrict__ out) {
  static_assert(QP == 1 || QP == 2, "one or two query pairs per pass");
  constexpr int W = 4 * T;
  constexpr int m = 32 * W;
  constexpr int NQ = 2 * QP;
  constexpr int JL = m / 64;
  __shared__ __attribute__((aligned(16))) unsigned char sAimg[QueryOperands<T, QP>::IMAGE_BYTES];
  __shared__ __attribute__((aligned(16))) float sPart[SM_WAVES][NQ][AT_PART];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = gridDim.x;
  // key positions within a group fit an int, and byte offsets into a
  // group's rows a uint32 (the fused path takes nk < 2^22).  The loads go
  // through descriptors over [kbeg, kend); the workgroup's stage i holds keys
  // key0 + kstride i + [0, AT_STAGE) of that range, which ends at nkb.  inter
  // = 0: a contiguous chunk of `chunk` keys; inter = 1: every P-th stage of
  // the whole group (the group's workgroups sweep its keys together).
  int kbeg, kend, key0, kstride, nstage_blk;
  if (inter) {
    const int nst = (int)((nk + AT_STAGE - 1) / AT_STAGE), x = (int)blockIdx.x;
    kbeg = 0;
    kend = (int)nk;
    key0 = AT_STAGE * x;
    kstride = AT_STAGE * P;
    nstage_blk = x < nst ? (nst - x + P - 1) / P : 0;
  } else {
    kbeg = (int)blockIdx.x * chunk;
    kend = (int64_t)kbeg + chunk < nk ? kbeg + chunk : (int)nk;
    key0 = 0;
    kstride = AT_STAGE;
    nstage_blk = ((kend > kbeg ? kend - kbeg : 0) + AT_STAGE - 1) / AT_STAGE;
  }
  const int nkb = kend > kbeg ? kend - kbeg : 0;  // keys of the descriptors' range
  const int ns = (nstage_blk - wave + SM_WAVES - 1) / SM_WAVES;
  constexpr int R = attn_ring<T, PAIR>();
  const int nsr = (ns + R - 1) / R * R;  // whole rounds of the ring

  for (int64_t g = blockIdx.y; g < G; g += gridDim.y) {
    const KeyRange kr = key_range<T>(bits + g * nk * (int64_t)W, norms + g * nk,
                                     V + g * nk * (int64_t)AT_DV, kbeg, kend);
    for (int64_t q0 = 0; q0 < nq; q0 += NQ) {
      const int nqp = (int)((nq - q0) < NQ ? (nq - q0) : NQ);
      float sv[NQ][JL];
      load_query_values<m, NQ>(Sq + (g * nq + q0) * (int64_t)m, nqp, lane, sv);
      // (the previous pass's merge barrier orders its image reads before
      // this image's writes)
      QueryOperands<T, QP> qo;
      build_query_operands<T, QP>(sv, nqp, wave, lane, sAimg, cscale, qo);
      __builtin_amdgcn_sched_barrier(0);
      AttnStage<T> ring[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        load_attn_stage<T>(ring[r], kr, key0 + kstride * (wave + SM_WAVES * r), lane);
      SoftmaxState<QP> st;
#pragma unroll
      for (int qp = 0; qp < QP; ++qp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          st.M[qp][h] = -INFINITY;
          st.L[qp][h] = 0.f;
#pragma unroll
          for (int d = 0; d < 8; ++d) st.acc[qp][h][d] = 0.f;
        }
      stream_keys<T, QP, PAIR, R>(ring, kr, qo, wave, lane, nsr, key0, kstride, nkb, nqp, sl2,
                                  st);
      // ---- this wave's partials: sum the four lane groups (each saw every
      // fourth value row); lanes 0..15 then hold dims 8 lane .. 8 lane + 7
#pragma unroll
      for (int qi = 0; qi < NQ; ++qi) {
        if (qi >= nqp) break;
        const int qp = qi >> 1, h = qi & 1;
        float a[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          a[d] = st.acc[qp][h][d];
          a[d] += __shfl_xor(a[d], 16);
          a[d] += __shfl_xor(a[d], 32);
        }
        float *dst = sPart[wave][qi];
        if (lane < 16) {
          reinterpret_cast<float4 *>(dst)[2 * lane] = make_float4(a[0], a[1], a[2], a[3]);
          reinterpret_cast<float4 *>(dst)[2 * lane + 1] = make_float4(a[4], a[5], a[6], a[7]);
        }
        if (lane == 0) {
          dst[AT_DV] = st.M[qp][h];
          dst[AT_DV + 1] = st.L[qp][h];
        }
      }
      __syncthreads();
      // ---- the workgroup's partial of query h, merged by wave h
      if (wave < nqp) {
        const int h = wave;
        float Mw[SM_WAVES], M = -INFINITY;
#pragma unroll
        for (int w = 0; w < SM_WAVES; ++w) {
          Mw[w] = sPart[w][h][AT_DV];
          M = fmaxf(M, Mw[w]);
        }
        float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int w = 0; w < SM_WAVES; ++w) {
          const float f = exp2_shift(Mw[w], M);
          L = fmaf(f, sPart[w][h][AT_DV + 1], L);
          o0 = fmaf(f, sPart[w][h][lane], o0);
          o1 = fmaf(f, sPart[w][h][lane + 64], o1);
        }
        if (P == 1) {
          // the group's only workgroup: its merged state is the result
          const float inv = 1.f / L;
          float *o = out + (g * nq + q0 + h) * (int64_t)AT_DV;
          o[lane] = o0 * inv;
          o[lane + 64] = o1 * inv;
        } else {
          float *dst = ws + ((g * nq + q0 + h) * (int64_t)P + blockIdx.x) * AT_PART;
          dst[lane] = o0;
          dst[lane + 64] = o1;
          if (lane == 0) {
            dst[AT_DV] = M;
            dst[AT_DV + 1] = L;
          }
        }
      }
      __syncthreads();  // sPart and the query image are free again
    }
  }
}

// Merge the P partials of each (group, query) row: M = max M_p,
// out = sum_p 2^(M_p - M) acc_p / sum_p 2^(M_p - M) L_p.  One wave per row:
// lane p reads the maximum and sum of partial p (64 partials per round),
// lane l sums dims l and l + 64 over the partials.
__global__ __launch_bounds__(64) void attn_combine_kernel(const float *__restrict__ ws,
                                                          int64_t rows, int P,
                                                          float *__restrict__ out) {
  const int lane = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const float *base = ws + row * (int64_t)P * AT_PART;
    float M = -INFINITY;
    for (int p = lane; p < P; p += 64) M = fmaxf(M, base[p * AT_PART + AT_DV]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p0 = 0; p0 < P; p0 += 64) {
      const int p = p0 + lane;
      const float f = p < P ? exp2_shift(base[p * AT_PART + AT_DV], M) : 0.f;
      L += p < P ? f * base[p * AT_PART + AT_DV + 1] : 0.f;
      const int n = P - p0 < 64 ? P - p0 : 64;
      int i = 0;
      for (; i + 4 <= n; i += 4) {  // four partials' loads in flight
        float a0[4], a1[4], fi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float *e = base + (p0 + i + u) * AT_PART;
          a0[u] = e[lane];
          a1[u] = e[lane + 64];
          fi[u] = __shfl(f, i + u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o0 = fmaf(fi[u], a0[u], o0);
          o1 = fmaf(fi[u], a1[u], o1);
        }
      }
      for (; i < n; ++i) {
        const float fi = __shfl(f, i);
        const float *e = base + (p0 + i) * AT_PART;
        o0 = fmaf(fi, e[lane], o0);
        o1 = fmaf(fi, e[lane + 64], o1);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
    const float inv = 1.f / L;
    out[row * AT_DV + lane] = o0 * inv;
    out[row * AT_DV + lane + 64] = o1 * inv;
  }
}

// Plain path: scores already in the workspace ([G * nq][nk]); one workgroup
// per (group, query) row.  Pass 1 finds the maximum, pass 2 forms the weights
// and the weighted sum, threads splitting the value dimensions.
template <typename TV>
__global__ __launch_bounds__(256) void attn_softmax_kernel(const float *__restrict__ scores,
                                                           const TV *__restrict__ V, int64_t rows,
                                                           int64_t nq, int64_t nk, int dv,
                                                           float sl2, float *__restrict__ out) {
  __shared__ float red[256];
  const int tid = threadIdx.x;
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t g = row / nq;
    const float *s = scores + row * nk;
    const TV *gv = V + g * nk * (int64_t)dv;
    float mx = -INFINITY;
    for (int64_t t = tid; t < nk; t += 256) mx = fmaxf(mx, s[t] * sl2);
    red[tid] = mx;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
      __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float l = 0.f;
    for (int64_t t = tid; t < nk; t += 256) l += exp2f(s[t] * sl2 - mx);
    red[tid] = l;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const float inv = 1.f / red[0];
    __syncthreads();
    for (int d = tid; d < dv; d += 256) {
      float o = 0.f;
      for (int64_t t = 0; t < nk; ++t) o = fmaf(exp2f(s[t] * sl2 - mx), load_as_f32(gv, t * dv + d), o);
      out[row * dv + d] = o * inv;
    }
  }
}

// The fast path's grid: one workgroup per compute unit over the keys of all
// groups, at most 65535 groups per launch row.
template <int T, int QP>
void attn_grid(int64_t G, int64_t nk, int64_t *chunk_out, int *gx_out) {
  // One workgroup per compute unit streams as fast as two (and, with fewer
  // partials, combines faster: long context 241 against 245 us).  With at
  // least one group per compute unit, each group gets one workgroup, which
  // writes the result itself with no combine pass (7B decode: 104 against
  // 111 us with two workgroups per unit and the combine).
  static PerDevice pd_cus;
  const int cus = per_device(pd_cus, device_compute_units);
  int64_t chunk = (G * nk + cus - 1) / cus;
  constexpr int round = 3 * AT_STAGE * SM_WAVES;  // whole rounds of a three-stage ring
  chunk = (chunk + round - 1) / round * round;
  if (G >= cus) chunk = (nk + round - 1) / round * round;
  *chunk_out = chunk;
  *gx_out = (int)((nk + chunk - 1) / chunk);
}

template <int T, int QP>
hipError_t launch_attn_t(const float *Sq, const uint32_t *bits, const float *norms,
                         const uint16_t *V, int64_t G, int64_t nq, int64_t nk, float c, float sl2,
                         float *ws, float *out, hipStream_t st) {
  int64_t chunk = 0;
  int gx = 0;
  attn_grid<T, QP>(G, nk, &chunk, &gx);
  const int P = gx;
  dim3 grid((unsigned)gx, (unsigned)(G < 65535 ? G : 65535));
  // A group's workgroups interleave its stages rather than take a chunk each.
  const int inter = P > 1 ? 1 : 0;
  if (nq > 1)
    hipLaunchKernelGGL((attn_partial_kernel<T, QP, true>), grid, dim3(SM_THREADS), 0, st, Sq,
                       bits, norms, V, G, nq, nk, (int)chunk, inter, c, sl2, ws, out);
  else
    hipLaunchKernelGGL((attn_partial_kernel<T, 1, false>), grid, dim3(SM_THREADS), 0, st, Sq,
                       bits, norms, V, G, nq, nk, (int)chunk, inter, c, sl2, ws, out);
  if (P > 1) {  // with one workgroup per group the kernel wrote the output itself
    const int64_t rows = G * nq;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(rows < 65535 ? rows : 65535)),
                       dim3(64), 0, st, ws, rows, P, out);
  }
  return hipGetLastError();
}

template <int T>
int attn_partials_t(int64_t G, int64_t nk) {
  int64_t chunk = 0;
  int gx = 0;
  attn_grid<T, 1>(G, nk, &chunk, &gx);
  return gx;
}

}  // namespace

// Sketch sizes with a fused instantiation (T = m / 128 words per lane group).
static bool fused_m(int m) { return m == 128 || m == 256 || m == 512 || m == 1024; }

hipError_t launch_attn_combine(const float *ws, int64_t rows, int P, float *out, hipStream_t st) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(rows < 65535 ? rows : 65535)), dim3(64),
                     0, st, ws, rows, P, out);
  return hipGetLastError();
}

// Whether the fused path serves this call (the rest takes the plain path).
bool attention_fused_supported(const qjl_sketch *sk, const uint32_t *bits, const void *V,
                               int v_dtype, int dv, int64_t nk) {
  const int m = sk->host.m;
  return v_dtype == QJL_DTYPE_BF16 && dv == AT_DV && fused_m(m) &&
         nk < (int64_t(1) << 22) && ((uintptr_t)bits & 15) == 0 && ((uintptr_t)V & 15) == 0;
}

size_t attention_workspace_bytes(const qjl_sketch *sk, int64_t G, int64_t nq, int64_t nk, int dv) {
  const int m = sk->host.m;
  size_t fused = 0;
  if (dv == AT_DV && fused_m(m) && nk < (int64_t(1) << 22)) {
    int P = 0;
    switch (m / 128) {
      case 1: P = attn_partials_t<1>(G, nk); break;
      case 2: P = attn_partials_t<2>(G, nk); break;
      case 4: P = attn_partials_t<4>(G, nk); break;
      case 8: P = attn_partials_t<8>(G, nk); break;
      default: P = 0;
    }
    if (attn_mq_supported(m / 128)) {
      const int Pm = attn_mq_partials(m / 128, G, nk);
      P = P > Pm ? P : Pm;
    }
    fused = (size_t)G * nq * P * AT_PART * sizeof(float);
  }
  const size_t plain = (size_t)G * nq * nk * sizeof(float);
  return fused > plain ? fused : plain;
}

hipError_t launch_attention_fused(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                  const float *norms, const void *V, int64_t G, int64_t nq,
                                  int64_t nk, float scale, float *ws, float *out,
                                  hipStream_t st) {
  const HostSketch &h = sk->host;
  const float c = estimator_scale(h.m, h.rho);
  const float sl2 = scale * LOG2E;
  const uint16_t *Vb = static_cast<const uint16_t *>(V);
  const int T = h.m / 128;
  // Three or more queries per group (grouped-query attention): up to eight
  // queries per pass, their weighted sums on the matrix cores.
  if (nq >= 3 && attn_mq_supported(T)) {
    int P = 0;
    hipError_t e =
        launch_attn_mq_partials(T, Sq, bits, norms, Vb, G, nq, nk, c, sl2, ws, out, &P, st);
    if (e != hipSuccess || P == 1) return e;
    return launch_attn_combine(ws, G * nq, P, out, st);
  }
  switch (T) {
    case 1: return launch_attn_t<1, 1>(Sq, bits, norms, Vb, G, nq, nk, c, sl2, ws, out, st);
    case 2: return launch_attn_t<2, 1>(Sq, bits, norms, Vb, G, nq, nk, c, sl2, ws, out, st);
    case 4: return launch_attn_t<4, 1>(Sq, bits, norms, Vb, G, nq, nk, c, sl2, ws, out, st);
    case 8: return launch_attn_t<8, 1>(Sq, bits, norms, Vb, G, nq, nk, c, sl2, ws, out, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention_softmax(const float *scores, const void *V, int v_dtype, int dv,
                                    int64_t G, int64_t nq, int64_t nk, float scale, float *out,
                                    hipStream_t st) {
  const int64_t rows = G * nq;
  const unsigned grid = (unsigned)(rows < 65535 ? rows : 65535);
  const float sl2 = scale * LOG2E;
  if (v_dtype == QJL_DTYPE_F32)
    hipLaunchKernelGGL(attn_softmax_kernel<float>, dim3(grid), dim3(256), 0, st, scores,
                       static_cast<const float *>(V), rows, nq, nk, dv, sl2, out);
  else
    hipLaunchKernelGGL(attn_softmax_kernel<uint16_t>, dim3(grid), dim3(256), 0, st, scores,
                       static_cast<const uint16_t *>(V), rows, nq, nk, dv, sl2, out);
  return hipGetLastError();
}

}  // namespace qjl
