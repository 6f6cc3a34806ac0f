// Internal declarations shared by the host API and the HIP kernels of libqjl.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "../../include/qjl.h"

namespace qjl {

// SplitMix64 output function (Steele, Lea & Flood, OOPSLA 2014) and the
// counter streams built on it:  key(seed, s) = mix64(seed + PHI (s + 1)),
// r(seed, s, i) = mix64(key + PHI (i + 1)).
constexpr uint64_t PHI = 0x9E3779B97F4A7C15ull;
__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}
__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed + PHI * (stream + 1));
}
__host__ __device__ inline uint64_t stream_draw(uint64_t key, uint64_t i) {
  return mix64(key + PHI * (i + 1));
}

// Streams: 0 dense S, 1 D, 2 P, 3 G, 4 dither magnitudes (per sketch),
// 5 dither signs (per key).
enum : int {
  STREAM_DENSE = 0,
  STREAM_D = 1,
  STREAM_P = 2,
  STREAM_G = 3,
  STREAM_DITHER = 4,
  STREAM_DITHER_SIGN = 5
};

// Output row of quantized key r in a cache laid out by group: key r is key
// r % per_group of group r / per_group and goes to row
// (r / per_group) * stride + first + r % per_group; its dither key index is
// key_index_base plus that row.  per_group == 0 is the identity (row r).
// The division is 32-bit: callers keep r below 2^32.
struct RowMap {
  int64_t per_group = 0, stride = 0, first = 0;
};
__host__ __device__ inline int64_t map_row(const RowMap &mp, int64_t r) {
  if (mp.per_group == 1) return r * mp.stride + mp.first;
  const uint32_t g = (uint32_t)r / (uint32_t)mp.per_group;
  return (int64_t)g * mp.stride + mp.first + (r - (int64_t)g * mp.per_group);
}

// Host-side random parameters of one sketch (no device state).
struct HostSketch {
  uint64_t seed = 0;
  int d = 0, m = 0, variant = 0;
  float rho = 0.f;
  std::vector<float> S32;      // dense: m*d, float32 rounding of the Gaussian draws
  std::vector<uint16_t> S16;   // dense: m*d, bfloat16 bits (RNE of S32)
  std::vector<int8_t> D;       // FQJL: nb*d, +1/-1
  std::vector<int32_t> P;      // FQJL: nb*d, permutation of [0, d) per block
  std::vector<float> G;        // FQJL: nb*d, float32 Gaussians
  std::vector<float> Dmag;     // m dither magnitudes fp32(|N(j)|), stream 4 (every variant)
};

qjl_status validate_sketch_params(int32_t d, int32_t m, int32_t variant, float rho,
                                  bool check_rho = true);
void generate_host_sketch(HostSketch &hs);
uint16_t f32_to_bf16_rne(float x);
// Explicit m x d FQJL matrix (double), for export.
void fqjl_explicit(const HostSketch &hs, std::vector<double> &out);

// Host-written operand images (images_host.cpp): the dense bf16 S in the
// matrix-core operand order (m * d values), and the FQJL first stage
// (m * d values, only for the shapes fqjl_mfma_image_shape accepts).
void build_mfma_b_layout(const uint16_t *S16, int d, int m, uint16_t *out);
bool fqjl_mfma_image_shape(int d, int m);
void build_fqjl_mfma_image(const HostSketch &hs, uint16_t *out);

}  // namespace qjl

// Device-resident sketch.  All device arrays live in one allocation `dmem`.
struct qjl_sketch {
  qjl::HostSketch host;
  int device = -1;
  uint64_t dither_key = 0;       // key(seed, 5): the stream of each key's dither signs
  void *dmem = nullptr;
  // dense
  const float *S32 = nullptr;    // m*d  float32 S (row-major)
  const float *S16f = nullptr;   // m*d  bfloat16-rounded S widened to float32 (row-major)
  const uint16_t *S16mfma = nullptr;  // m*d bf16 in the MFMA B-operand order (see k_quantize_mfma)
  const float *S32T = nullptr;   // d*m  float32 S transposed (column j of row c at c*m + j)
  const float *S16fT = nullptr;  // d*m  bfloat16-rounded S transposed, widened to float32
  // FQJL
  const uint32_t *Dsign = nullptr;    // nb*d sign masks: 0 (D=+1) or 0x80000000 (D=-1)
  const int32_t *P = nullptr;         // nb*d
  const float *Gs = nullptr;          // nb*d  G_b[c] / sqrt(d), rounded to float32
  const uint16_t *Fmfma = nullptr;    // m*d bf16 (+-1): Pi_b H diag(D_b) in matrix-core operand
                                      // order (k_fqjl_mfma), for d = 128; null otherwise
  // every variant
  const float *Dmag = nullptr;        // m  dither magnitudes |N(j)| (float32)
};

namespace qjl {

// Kernel launchers (each returns hipGetLastError() of its launch).
hipError_t launch_quantize_generic(const qjl_sketch *sk, const void *K, int dtype, int64_t n,
                                   int64_t base, const RowMap &map, float *norms, uint32_t *bits,
                                   hipStream_t st);
hipError_t launch_project_dense(const qjl_sketch *sk, const void *q, int dtype, int64_t n,
                                float *Sq, hipStream_t st);
bool project_mfma_supported(const qjl_sketch *sk, const void *q, int dtype, int64_t n,
                            const float *Sq);
hipError_t launch_project_mfma(const qjl_sketch *sk, const void *q, int64_t n, float *Sq,
                               hipStream_t st);
bool quantize_mfma_supported(const qjl_sketch *sk, const void *K, int dtype,
                             const uint32_t *bits);
hipError_t launch_quantize_mfma(const qjl_sketch *sk, const void *K, int64_t n, const RowMap &map,
                                float *norms, uint32_t *bits, hipStream_t st);
bool fqjl_mfma_supported(const qjl_sketch *sk, const void *K, int dtype, const uint32_t *bits);
hipError_t launch_fqjl_mfma(const qjl_sketch *sk, const void *K, int64_t n, int64_t base,
                            const RowMap &map, float *norms, uint32_t *bits, hipStream_t st);
bool fqjl_project_mfma_supported(const qjl_sketch *sk, const void *q, int dtype, const float *Y);
hipError_t launch_fqjl_project_mfma(const qjl_sketch *sk, const void *q, int64_t n, float *Y,
                                    hipStream_t st);
hipError_t launch_fqjl(const qjl_sketch *sk, const void *X, int dtype, int64_t n, int64_t base,
                       const RowMap &map, float *norms, uint32_t *bits, float *Y, hipStream_t st);
hipError_t launch_score_generic(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, int64_t G, int64_t nq, int64_t nk,
                                float *scores, hipStream_t st);
hipError_t launch_score(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                        const float *norms, int64_t G, int64_t nq, int64_t nk, float *scores,
                        hipStream_t st);

// Decode attention (k_attention.hip).
bool attention_fused_supported(const qjl_sketch *sk, const uint32_t *bits, const void *V,
                               int v_dtype, int dv, int64_t nk);
size_t attention_workspace_bytes(const qjl_sketch *sk, int64_t G, int64_t nq, int64_t nk, int dv);
hipError_t launch_attention_fused(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                  const float *norms, const void *V, int64_t G, int64_t nq,
                                  int64_t nk, float scale, float *ws, float *out, hipStream_t st);
hipError_t launch_attention_softmax(const float *scores, const void *V, int v_dtype, int dv,
                                    int64_t G, int64_t nq, int64_t nk, float scale, float *out,
                                    hipStream_t st);

// Host-computed data the score kernels take per launch.
float estimator_scale(int m, float rho);

// qjl_decode_attention's argument checks other than the workspace (pointers,
// counts, dtype, alignment, the sketch's device), shared with the
// allocation-free variant; *noop is set when there is nothing to compute.
qjl_status attention_check_args(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                                int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                                float softmax_scale, const float *out, bool *noop);
// Enqueue the decode attention with `ws` as its workspace (at least
// attention_workspace_bytes, 16-byte aligned; checked by the caller).
qjl_status attention_run(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                         const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                         int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                         float softmax_scale, float *ws, float *out, void *stream);

}  // namespace qjl
