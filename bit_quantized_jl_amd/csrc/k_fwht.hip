// FQJL sketch kernel: stacked blocks H diag(G_b) Pi_b (H/sqrt d) diag(D_b)
// ("Fast Quantized Johnson-Lindenstrauss Transforms" page: randomized
// Hadamard transforms with a Gaussian second diagonal and a uniform random
// permutation between them; optional Gaussian dither before the sign).
//
// One row (key or query) per lane.  The d coordinates of a row live in the
// lane's registers, so both Walsh-Hadamard transforms are unrolled butterfly
// networks with no cross-lane traffic (O(d log d) additions per block).  The
// permutation is the only data-dependent step: each lane stores its vector to
// its own column of an LDS tile (element c at c*64 + lane, which is bank-
// conflict free because the 64 lanes hit consecutive words) and gathers it
// back in the order P_b.  A lane reads only what it wrote, so no barrier is
// needed.  Sign bits are packed per lane into 32-bit words (bit = [y >= 0],
// which maps -0 to 1 like +0).  All arithmetic is float32.
//
// Coordinates: block b produces sketch coordinates [b d, (b+1) d).  G_b is
// pre-scaled by 1/sqrt(d) on the host, so the kernel computes
// H (Gs_b * (H (D_b x))[P_b]).
//
// These all-vector kernels serve projections, float32 keys, d < 128,
// d = 256 (fqjl256_kernel: four lanes per row) and buffers that are not
// 16-byte aligned; bfloat16 keys at d = 128 are quantized by k_fqjl_mfma.hip,
// which applies the first stage on the matrix cores (launch_fqjl routes them).
#include "device_common.h"
#include "fwht_common.h"

namespace qjl {

namespace {

// Row loads as 16-byte vectors (a 2-byte load per element leaves each load
// instruction touching 64 cache lines for 128 bytes).
template <int D, typename T>
__device__ __forceinline__ void load_row_vec(const T *__restrict__ xr, bool valid, float (&x)[D]) {
  const uint4 *src = reinterpret_cast<const uint4 *>(xr);
  constexpr int NV = D * (int)sizeof(T) / 16;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint4 q = src[v];
    const uint32_t w[4] = {valid ? q.x : 0u, valid ? q.y : 0u, valid ? q.z : 0u, valid ? q.w : 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 4) {
        x[4 * v + e] = __uint_as_float(w[e]);
      } else {
        x[8 * v + 2 * e] = __uint_as_float(w[e] << 16);
        x[8 * v + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
}

// PERM = false: the block has no permutation (D-FQJL), so the transformed
// row is scaled by G in place and the LDS round trip is skipped.
template <int D, typename T, bool PROJECT, bool DITHER, bool VEC, bool PERM, bool MAPPED>
__global__ __launch_bounds__(64) void fqjl_kernel(
    const T *__restrict__ X, int nb, int m, const uint32_t *__restrict__ Dsign,
    const int32_t *__restrict__ P, const float *__restrict__ Gs, int64_t n, int64_t base,
    RowMap map, float rho, uint64_t dkey, const float *__restrict__ Dmag,
    float *__restrict__ norms, uint32_t *__restrict__ bits,
    float *__restrict__ Y) {
  __shared__ float lds[D * 64];
  const int lane = threadIdx.x;
  const int W = m / 32;
  constexpr bool HOLD = true;  // keep the input row in registers across blocks
  for (int64_t r0 = (int64_t)blockIdx.x * 64; r0 < n; r0 += (int64_t)gridDim.x * 64) {
    const int64_t row = r0 + lane;
    const bool valid = row < n;
    const int64_t orow = MAPPED ? map_row(map, valid ? row : 0) : (valid ? row : 0);  // output row
    const T *xr = X + (valid ? row : 0) * (int64_t)D;
    float x[HOLD ? D : 1];
    float nrm = 0.f;
    if (HOLD) {
      if constexpr (VEC) {
        load_row_vec<D, T>(xr, valid, x);
      } else {
#pragma unroll
        for (int c = 0; c < D; ++c) x[c] = valid ? load_as_f32(xr, c) : 0.f;
      }
    }
    if (!PROJECT) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        const float v = HOLD ? x[c] : (valid ? load_as_f32(xr, c) : 0.f);
        s = fmaf(v, v, s);
      }
      nrm = sqrtf(s);
      if (valid) norms[orow] = nrm;
    }
    for (int b = 0; b < nb; ++b) {
      float u[D];
      const uint32_t *ds = Dsign + b * D;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        const float v = HOLD ? x[c] : (valid ? load_as_f32(xr, c) : 0.f);
        u[c] = __uint_as_float(__float_as_uint(v) ^ ds[c]);
      }
      fwht_reg<D>(u);
      const int32_t *pb = P + b * D;
      const float *gb = Gs + b * D;
      if constexpr (PERM) {
#pragma unroll
        for (int c = 0; c < D; ++c) lds[c * 64 + lane] = u[c];
#pragma unroll
        for (int c = 0; c < D; ++c) u[c] = lds[pb[c] * 64 + lane] * gb[c];
      } else {
#pragma unroll
        for (int c = 0; c < D; ++c) u[c] *= gb[c];
      }
      fwht_reg<D>(u);
      if (PROJECT) {
        if (valid) {
          float *yr = Y + row * (int64_t)m + b * D;
#pragma unroll
          for (int c = 0; c < D; ++c) yr[c] = u[c];
        }
      } else {
        if (DITHER)
          dither_words_add<D / 32>(u, rho * nrm, dkey, (uint64_t)(base + orow), m, b * D / 32,
                                   Dmag + b * D);
        if (valid) {
          uint32_t *br = bits + orow * (int64_t)W + b * (D / 32);
#pragma unroll
          for (int w = 0; w < D / 32; ++w) br[w] = pack_nonneg(&u[32 * w]);
        }
      }
    }
  }
}

// d = 128 with two lanes per row (32 rows per wave): lane half s computes
// output half s of each Walsh-Hadamard transform.  H_128 = [[H, H], [H, -H]]
// with H = H_64, so half s of H_128 z is H_64 (z_lo + (-1)^s z_hi): each lane
// folds the top butterfly stage into how it combines its inputs and runs a
// 64-point transform, with no cross-lane exchange.  The permutation tile is
// then 16 KB per wave (element c of row k at ((c ^ (c >> 6)) << 5) + k: the
// two halves' writes land in disjoint banks, and every gather reads one index
// for all lanes, so it is conflict free), which doubles the waves a CU holds.
// Without a permutation (PERM = false, D-FQJL) each lane needs coordinate c
// of both halves, which v_permlane32_swap exchanges between lanes k and
// k + 32 in registers: no LDS at all.
template <typename T, bool PROJECT, bool DITHER, bool PERM, bool MAPPED>
__global__ __launch_bounds__(64, sizeof(T) == 2 ? 2 : 1) void fqjl128_kernel(
    const T *__restrict__ X, int nb, int m, const uint32_t *__restrict__ Dsign,
    const int32_t *__restrict__ P, const float *__restrict__ Gs, int64_t n, int64_t base,
    RowMap map, float rho, uint64_t dkey, const float *__restrict__ Dmag,
    float *__restrict__ norms, uint32_t *__restrict__ bits,
    float *__restrict__ Y) {
  constexpr int D = 128, H = 64;
  __shared__ float lds[D * 32];
  const int lane = threadIdx.x;
  const int k = lane & 31, sh = lane >> 5;
  const float sgn = sh ? -1.f : 1.f;
  const int W = m / 32;
  auto idx = [](int c, int key) { return ((c ^ (c >> 6)) << 5) + key; };
  for (int64_t r0 = (int64_t)blockIdx.x * 32; r0 < n; r0 += (int64_t)gridDim.x * 32) {
    const int64_t row = r0 + k;
    const bool valid = row < n;
    const int64_t orow = MAPPED ? map_row(map, valid ? row : 0) : (valid ? row : 0);  // output row
    const T *xr = X + (valid ? row : 0) * (int64_t)D;
    // The row stays in registers as loaded (bf16 pairs or float words) and is
    // widened where it is used: half the registers of a float copy for bf16.
    constexpr int NW = D * (int)sizeof(T) / 4;
    uint32_t xw[NW];
    {
      const uint4 *src = reinterpret_cast<const uint4 *>(xr);
#pragma unroll
      for (int v = 0; v < NW / 4; ++v) {  // a row past n re-reads row 0 and stores nothing
        const uint4 q = src[v];
        xw[4 * v] = q.x;
        xw[4 * v + 1] = q.y;
        xw[4 * v + 2] = q.z;
        xw[4 * v + 3] = q.w;
      }
    }
    // Float bits of element c with its sign flipped by sm (0 or the sign
    // bit).  For an even bf16 element the flip is an add, which carries out of
    // bit 31 and so equals the xor: one v_lshl_add_u32 widens and flips.
    auto elem_flip = [&](int c, uint32_t sm) -> uint32_t {
      if constexpr (sizeof(T) == 4) return xw[c] ^ sm;
      else return (c & 1) ? ((xw[c >> 1] & 0xFFFF0000u) ^ sm) : ((xw[c >> 1] << 16) + sm);
    };
    float nrm = 0.f;
    if (!PROJECT) {  // each lane half sums half the row, one selected word at a time
      float ssq = 0.f;
#pragma unroll
      for (int i = 0; i < NW / 2; ++i) {
        const uint32_t w = sh ? xw[i + NW / 2] : xw[i];
        if constexpr (sizeof(T) == 4) {
          ssq = fmaf(__uint_as_float(w), __uint_as_float(w), ssq);
        } else {
          const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
          ssq = fmaf(lo, lo, ssq);
          ssq = fmaf(hi, hi, ssq);
        }
      }
      nrm = sqrtf(ssq + __shfl_xor(ssq, 32));
      if (valid && sh == 0 && blockIdx.y == 0) norms[orow] = nrm;
    }
    // blocks b = blockIdx.y, blockIdx.y + gridDim.y, ...: a short call (few
    // rows, e.g. one new key per head) spreads its blocks over workgroups
    for (int b = blockIdx.y; b < nb; b += gridDim.y) {
      // Re-widen the row inside each block: hoisted out of this loop, the
      // widened copy would sit in registers beside the packed one.
#pragma unroll
      for (int i = 0; i < NW; ++i) asm volatile("" : "+v"(xw[i]));
      const uint32_t *ds = Dsign + b * D;
      const int32_t *pb = P + b * D;
      const float *gb = Gs + b * D;
      float t[H];
#pragma unroll
      for (int c = 0; c < H; ++c) {
        const float lo = __uint_as_float(elem_flip(c, ds[c]));
        const float hi = __uint_as_float(elem_flip(c + H, ds[c + H]));
        t[c] = fmaf(sgn, hi, lo);
      }
      fwht_reg<H>(t);
      if constexpr (PERM) {
        {
          // idx(c + 64 sh, k) = 32 (c ^ sh) + 2048 sh + k for c < 64: one lane base
          // for even and one for odd c, plus an immediate offset 32 c.
          float *we = lds + k + 2048 * sh + 32 * sh;
          float *wo = lds + k + 2048 * sh - 32 * sh;
#pragma unroll
          for (int c = 0; c < H; ++c) ((c & 1) ? wo : we)[32 * c] = t[c];
        }
        // Gather in groups of 16: the barriers keep the compiler from hoisting
        // all 128 reads (and their addresses) into registers at once.
#pragma unroll
        for (int c = 0; c < H; ++c) {
          if (c % 16 == 0) asm volatile("" ::: "memory");
          const float lo = lds[idx(pb[c], k)] * gb[c];
          const float hi = lds[idx(pb[c + H], k)] * gb[c + H];
          t[c] = fmaf(sgn, hi, lo);
        }
      } else {
        // t[c] is coordinate c + 64 sh of the transformed row; after the swap
        // every lane holds coordinate c of half 0 (first) and half 1 (second)
#pragma unroll
        for (int c = 0; c < H; ++c) {
          const uint32_t v = __float_as_uint(t[c]);
          const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
          const float lo = __uint_as_float(sw[0]) * gb[c];
          const float hi = __uint_as_float(sw[1]) * gb[c + H];
          t[c] = fmaf(sgn, hi, lo);
        }
      }
      fwht_reg<H>(t);
      const int j0 = b * D + H * sh;  // sketch coordinate of t[0]
      if (PROJECT) {
        if (valid) {
          float *yr = Y + row * (int64_t)m + j0;
#pragma unroll
          for (int c = 0; c < H; ++c) yr[c] = t[c];
        }
      } else {
        if (DITHER)
          dither_words_add<H / 32>(t, rho * nrm, dkey, (uint64_t)(base + orow), m, j0 / 32,
                                   Dmag + j0);
        if (valid) {
          uint32_t *br = bits + orow * (int64_t)W + j0 / 32;
#pragma unroll
          for (int w = 0; w < H / 32; ++w) br[w] = pack_nonneg(&t[32 * w]);
        }
      }
    }
  }
}

// d = 256 with four lanes per row (16 rows per wave).  Sylvester order puts
// the quarter index in the top two bits of a coordinate, so H_256 = H_4 (x)
// H_64: quarter s of H_256 z is H_64 (sum_t H_4[s][t] z_t), z_t the t-th 64
// coordinates.  Lane quarter s (lanes 16 s .. 16 s + 15, one row each) holds
// z_s; the H_4 mix is two butterfly stages across the quarters,
// v_permlane16_swap of a value with itself handing every lane the values of
// quarters s & ~1 and s | 1, v_permlane32_swap those of s & ~2 and s | 2.
// Then each lane runs a 64-point transform on its own registers.  The
// permutation goes through a 16 KB LDS tile (element c of row k at
// 16 (c ^ (c >> 6)) + k, so the four quarters' writes land in distinct
// banks); each lane gathers its own quarter of the permuted, Gaussian-scaled
// row and the second transform repeats the first's pattern.  A row's
// quarters are read by the four lanes that own it, so every register holds
// 64 coordinates and the row is loaded once.
template <typename T, bool PROJECT, bool DITHER, bool VEC, bool PERM, bool MAPPED>
__global__ __launch_bounds__(64) void fqjl256_kernel(
    const T *__restrict__ X, int nb, int m, const uint32_t *__restrict__ Dsign,
    const int32_t *__restrict__ P, const float *__restrict__ Gs, int64_t n, int64_t base,
    RowMap map, float rho, uint64_t dkey, const float *__restrict__ Dmag,
    float *__restrict__ norms, uint32_t *__restrict__ bits,
    float *__restrict__ Y) {
  constexpr int D = 256, H = 64;
  __shared__ float lds[D * 16];
  const int lane = threadIdx.x;
  const int k = lane & 15, s = lane >> 4;
  const float sg0 = (s & 1) ? -1.f : 1.f;  // H_4 sign of this quarter, bit 0
  const float sg1 = (s & 2) ? -1.f : 1.f;  // and bit 1
  const int W = m / 32;
  // H_4 across the quarters, in place: t_s <- sum_u H_4[s][u] t_u.
  auto h4_mix = [&](float (&t)[H]) {
#pragma unroll
    for (int c = 0; c < H; ++c) {
      const uint32_t v = __float_as_uint(t[c]);
      const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      const uint32_t x = __float_as_uint(fmaf(sg0, __uint_as_float(a[1]), __uint_as_float(a[0])));
      const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
      t[c] = fmaf(sg1, __uint_as_float(b[1]), __uint_as_float(b[0]));
    }
  };
  for (int64_t r0 = (int64_t)blockIdx.x * 16; r0 < n; r0 += (int64_t)gridDim.x * 16) {
    const int64_t row = r0 + k;
    const bool valid = row < n;
    const int64_t orow = MAPPED ? map_row(map, valid ? row : 0) : (valid ? row : 0);  // output row
    const T *xr = X + (valid ? row : 0) * (int64_t)D + H * s;  // this lane's quarter
    float x[H];
    if constexpr (VEC) {
      load_row_vec<H, T>(xr, valid, x);
    } else {
#pragma unroll
      for (int c = 0; c < H; ++c) x[c] = valid ? load_as_f32(xr, c) : 0.f;
    }
    float nrm = 0.f;
    if (!PROJECT) {
      float ssq = 0.f;
#pragma unroll
      for (int c = 0; c < H; ++c) ssq = fmaf(x[c], x[c], ssq);
      ssq += __shfl_xor(ssq, 16);
      ssq += __shfl_xor(ssq, 32);
      nrm = sqrtf(ssq);
      if (valid && s == 0 && blockIdx.y == 0) norms[orow] = nrm;
    }
    // blocks b = blockIdx.y, blockIdx.y + gridDim.y, ...: a short call
    // spreads its blocks over workgroups
    for (int b = blockIdx.y; b < nb; b += gridDim.y) {
      const uint32_t *ds = Dsign + b * D + H * s;
      const int32_t *pb = P + b * D + H * s;
      const float *gb = Gs + b * D + H * s;
      float t[H];
#pragma unroll
      for (int c = 0; c < H; ++c) t[c] = __uint_as_float(__float_as_uint(x[c]) ^ ds[c]);
      h4_mix(t);
      fwht_reg<H>(t);
      if constexpr (PERM) {
#pragma unroll
        for (int c = 0; c < H; ++c) {
          const int e = H * s + c;
          lds[((e ^ (e >> 6)) << 4) + k] = t[c];
        }
        // Gather in groups of 16 (as in fqjl128_kernel: keeps the compiler
        // from hoisting every read and its address at once).
#pragma unroll
        for (int c = 0; c < H; ++c) {
          if (c % 16 == 0) asm volatile("" ::: "memory");
          const int e = pb[c];
          t[c] = lds[((e ^ (e >> 6)) << 4) + k] * gb[c];
        }
      } else {
#pragma unroll
        for (int c = 0; c < H; ++c) t[c] *= gb[c];
      }
      h4_mix(t);
      fwht_reg<H>(t);
      const int j0 = b * D + H * s;  // sketch coordinate of t[0]
      if (PROJECT) {
        if (valid) {
          float *yr = Y + row * (int64_t)m + j0;
#pragma unroll
          for (int c = 0; c < H; ++c) yr[c] = t[c];
        }
      } else {
        if (DITHER)
          dither_words_add<H / 32>(t, rho * nrm, dkey, (uint64_t)(base + orow), m, j0 / 32,
                                   Dmag + j0);
        if (valid) {
          uint32_t *br = bits + orow * (int64_t)W + j0 / 32;
          br[0] = pack_nonneg(&t[0]);
          br[1] = pack_nonneg(&t[32]);
        }
      }
    }
  }
}

// d = 8 or 16: a block is narrower than one 32-bit word, so the bits of
// consecutive blocks share words.  These small sizes exist so the GPU chain
// can be checked against explicit matrices; they run a plain per-lane loop
// that writes whole words after all blocks of a word are done.
template <int D, typename T, bool PROJECT, bool DITHER, bool MAPPED>
__global__ __launch_bounds__(64) void fqjl_small_kernel(
    const T *__restrict__ X, int nb, int m, const uint32_t *__restrict__ Dsign,
    const int32_t *__restrict__ P, const float *__restrict__ Gs, int64_t n, int64_t base,
    RowMap map, float rho, uint64_t dkey, const float *__restrict__ Dmag,
    float *__restrict__ norms, uint32_t *__restrict__ bits,
    float *__restrict__ Y) {
  const int lane = threadIdx.x;
  const int W = m / 32;
  for (int64_t r0 = (int64_t)blockIdx.x * 64; r0 < n; r0 += (int64_t)gridDim.x * 64) {
    const int64_t row = r0 + lane;
    if (row >= n) continue;
    const int64_t orow = MAPPED ? map_row(map, row) : row;  // output row
    float x[D];
#pragma unroll
    for (int c = 0; c < D; ++c) x[c] = load_as_f32(X + row * (int64_t)D, c);
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) s = fmaf(x[c], x[c], s);
    const float nrm = sqrtf(s);
    if (!PROJECT) norms[orow] = nrm;
    uint32_t word = 0;
    for (int b = 0; b < nb; ++b) {
      float u[D], v[D];
#pragma unroll
      for (int c = 0; c < D; ++c) u[c] = __uint_as_float(__float_as_uint(x[c]) ^ Dsign[b * D + c]);
      fwht_reg<D>(u);
      for (int c = 0; c < D; ++c) {
        // gather u[P[c]] from registers with a select chain (D <= 16)
        const int p = P[b * D + c];
        float g = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) g = (e == p) ? u[e] : g;
        v[c] = g * Gs[b * D + c];
      }
      fwht_reg<D>(v);
      for (int c = 0; c < D; ++c) {
        const int j = b * D + c;
        float y = v[c];
        if (PROJECT) {
          Y[row * (int64_t)m + j] = y;
          continue;
        }
        if (DITHER)
          y = dither_fma(y, rho * nrm, dither_word(dkey, (uint64_t)(base + orow), m, j >> 5),
                         j & 31, Dmag[j]);
        word |= (y >= 0.f ? 1u : 0u) << (j & 31);
        if ((j & 31) == 31) {
          bits[orow * (int64_t)W + (j >> 5)] = word;
          word = 0;
        }
      }
    }
  }
}

// Launch helpers: the boolean template arguments are chosen at run time.
struct FqjlArgs {
  int nb, m;
  const uint32_t *Dsign;
  const int32_t *P;
  const float *Gs;
  int64_t n, base;
  RowMap map;
  float rho;
  uint64_t dkey;
  const float *Dmag;
  float *norms;
  uint32_t *bits;
  float *Y;
};

template <typename T, bool PROJECT, bool DITHER, bool PERM>
void launch_fqjl128(const T *X, const FqjlArgs &a, dim3 grid, hipStream_t st) {
  if (!PROJECT && a.map.per_group != 0)
    hipLaunchKernelGGL((fqjl128_kernel<T, PROJECT, DITHER, PERM, true>), grid, dim3(64), 0, st,
                       X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
  else
    hipLaunchKernelGGL((fqjl128_kernel<T, PROJECT, DITHER, PERM, false>), grid, dim3(64), 0, st,
                       X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
}

template <typename T, bool PROJECT, bool DITHER, bool VEC, bool PERM>
void launch_fqjl256(const T *X, const FqjlArgs &a, dim3 grid, hipStream_t st) {
  if (!PROJECT && a.map.per_group != 0)
    hipLaunchKernelGGL((fqjl256_kernel<T, PROJECT, DITHER, VEC, PERM, true>), grid, dim3(64), 0,
                       st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
  else
    hipLaunchKernelGGL((fqjl256_kernel<T, PROJECT, DITHER, VEC, PERM, false>), grid, dim3(64), 0,
                       st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
}

template <typename T, bool VEC>
void launch_fqjl256_cases(const T *X, const FqjlArgs &a, bool proj, bool dith, bool perm,
                          dim3 grid, hipStream_t st) {
  if (!perm && proj) launch_fqjl256<T, true, false, VEC, false>(X, a, grid, st);
  else if (!perm && dith) launch_fqjl256<T, false, true, VEC, false>(X, a, grid, st);
  else if (proj) launch_fqjl256<T, true, false, VEC, true>(X, a, grid, st);
  else if (dith) launch_fqjl256<T, false, true, VEC, true>(X, a, grid, st);
  else launch_fqjl256<T, false, false, VEC, true>(X, a, grid, st);
}

template <int D, typename T, bool PROJECT, bool DITHER, bool VEC, bool PERM>
void launch_fqjl_row(const T *X, const FqjlArgs &a, int grid, hipStream_t st) {
  if (!PROJECT && a.map.per_group != 0)
    hipLaunchKernelGGL((fqjl_kernel<D, T, PROJECT, DITHER, VEC, PERM, true>), dim3(grid),
                       dim3(64), 0, st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map,
                       a.rho, a.dkey, a.Dmag, a.norms, a.bits, a.Y);
  else
    hipLaunchKernelGGL((fqjl_kernel<D, T, PROJECT, DITHER, VEC, PERM, false>), dim3(grid),
                       dim3(64), 0, st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map,
                       a.rho, a.dkey, a.Dmag, a.norms, a.bits, a.Y);
}

template <int D, typename T, bool PROJECT, bool DITHER>
void launch_fqjl_small(const T *X, const FqjlArgs &a, int grid, hipStream_t st) {
  if (!PROJECT && a.map.per_group != 0)
    hipLaunchKernelGGL((fqjl_small_kernel<D, T, PROJECT, DITHER, true>), dim3(grid), dim3(64), 0,
                       st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
  else
    hipLaunchKernelGGL((fqjl_small_kernel<D, T, PROJECT, DITHER, false>), dim3(grid), dim3(64), 0,
                       st, X, a.nb, a.m, a.Dsign, a.P, a.Gs, a.n, a.base, a.map, a.rho, a.dkey, a.Dmag,
                       a.norms, a.bits, a.Y);
}

// The PROJECT / DITHER / PERM combinations that occur: a projection never
// dithers, and a D-FQJL sketch (no permutation) always dithers its keys.
template <int D, typename T, bool VEC>
void launch_fqjl_rows(const T *X, const FqjlArgs &a, bool proj, bool dith, bool perm, int grid,
                      hipStream_t st) {
  if (!perm && proj) launch_fqjl_row<D, T, true, false, VEC, false>(X, a, grid, st);
  else if (!perm && dith) launch_fqjl_row<D, T, false, true, VEC, false>(X, a, grid, st);
  else if (proj) launch_fqjl_row<D, T, true, false, VEC, true>(X, a, grid, st);
  else if (dith) launch_fqjl_row<D, T, false, true, VEC, true>(X, a, grid, st);
  else launch_fqjl_row<D, T, false, false, VEC, true>(X, a, grid, st);
}

template <int D, typename T>
hipError_t launch_fqjl_t(const qjl_sketch *sk, const T *X, int64_t n, int64_t base,
                         const RowMap &map, float *norms, uint32_t *bits, float *Y,
                         hipStream_t st) {
  const HostSketch &h = sk->host;
  const FqjlArgs a{h.m / D, h.m, sk->Dsign, sk->P, sk->Gs, n, base, map, h.rho,
                   sk->dither_key, sk->Dmag, norms, bits, Y};
  const int64_t tiles = (n + 63) / 64;
  const int grid = (int)(tiles < 16384 ? tiles : 16384);
  const bool proj = Y != nullptr;
  const bool dith = !proj && h.rho > 0.f;
  // D-FQJL blocks have no permutation (P_b = I): the kernels skip the gather.
  // Any other case (P-FQJL, the composition) gathers through LDS.
  const bool perm = h.variant != QJL_VARIANT_DFQJL;
  if constexpr (D == 128) {
    if (((uintptr_t)X & 15) == 0) {  // rows are whole 16-byte vectors
      const int64_t tiles2 = (n + 31) / 32;
      const int grid2 = (int)(tiles2 < 32768 ? tiles2 : 32768);
      // Few rows: one workgroup per (row tile, block) so the blocks run side
      // by side (a row is then loaded once per block instead of once).
      const dim3 g2(grid2, tiles2 * a.nb <= 4096 ? a.nb : 1);
      if (!perm && proj) launch_fqjl128<T, true, false, false>(X, a, g2, st);
      else if (!perm && dith) launch_fqjl128<T, false, true, false>(X, a, g2, st);
      else if (proj) launch_fqjl128<T, true, false, true>(X, a, g2, st);
      else if (dith) launch_fqjl128<T, false, true, true>(X, a, g2, st);
      else launch_fqjl128<T, false, false, true>(X, a, g2, st);
      return hipGetLastError();
    }
  }
  if constexpr (D == 256) {
    const int64_t tiles4 = (n + 15) / 16;
    const int grid4 = (int)(tiles4 < 32768 ? tiles4 : 32768);
    // Few rows: one workgroup per (row tile, block), as for d = 128.
    const dim3 g4(grid4, tiles4 * a.nb <= 4096 ? a.nb : 1);
    if (((uintptr_t)X & 15) == 0)  // each quarter row is whole 16-byte vectors
      launch_fqjl256_cases<T, true>(X, a, proj, dith, perm, g4, st);
    else
      launch_fqjl256_cases<T, false>(X, a, proj, dith, perm, g4, st);
    return hipGetLastError();
  }
  if constexpr (D >= 32 && D <= 128) {
    if (((uintptr_t)X & 15) == 0)  // rows are whole 16-byte vectors
      launch_fqjl_rows<D, T, true>(X, a, proj, dith, perm, grid, st);
    else
      launch_fqjl_rows<D, T, false>(X, a, proj, dith, perm, grid, st);
  } else {
    if (proj) launch_fqjl_small<D, T, true, false>(X, a, grid, st);
    else if (dith) launch_fqjl_small<D, T, false, true>(X, a, grid, st);
    else launch_fqjl_small<D, T, false, false>(X, a, grid, st);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fqjl_d(const qjl_sketch *sk, const T *X, int64_t n, int64_t base,
                         const RowMap &map, float *norms, uint32_t *bits, float *Y,
                         hipStream_t st) {
  switch (sk->host.d) {
    case 8: return launch_fqjl_t<8>(sk, X, n, base, map, norms, bits, Y, st);
    case 16: return launch_fqjl_t<16>(sk, X, n, base, map, norms, bits, Y, st);
    case 32: return launch_fqjl_t<32>(sk, X, n, base, map, norms, bits, Y, st);
    case 64: return launch_fqjl_t<64>(sk, X, n, base, map, norms, bits, Y, st);
    case 128: return launch_fqjl_t<128>(sk, X, n, base, map, norms, bits, Y, st);
    case 256: return launch_fqjl_t<256>(sk, X, n, base, map, norms, bits, Y, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fqjl(const qjl_sketch *sk, const void *X, int dtype, int64_t n, int64_t base,
                       const RowMap &map, float *norms, uint32_t *bits, float *Y, hipStream_t st) {
  // bf16 keys at d = 128: the first stage on the matrix cores (k_fqjl_mfma),
  // for every row count.  Its short-call and persistent kernels form the
  // same sums in the same order, so a cache filled by appends is
  // bit-identical to one call over the whole cache; the kernels below sum
  // in another order and would not be.
  if (Y == nullptr && fqjl_mfma_supported(sk, X, dtype, bits))
    return launch_fqjl_mfma(sk, X, n, base, map, norms, bits, st);
  if (dtype == QJL_DTYPE_F32)
    return launch_fqjl_d(sk, static_cast<const float *>(X), n, base, map, norms, bits, Y, st);
  return launch_fqjl_d(sk, static_cast<const uint16_t *>(X), n, base, map, norms, bits, Y, st);
}

}  // namespace qjl
