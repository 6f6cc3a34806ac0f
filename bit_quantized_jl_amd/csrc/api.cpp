// extern "C" entry points of libqjl: validation, sketch lifetime, dispatch.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "qjl_internal.h"

using namespace qjl;

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

qjl_status check_device(const qjl_sketch *sk) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QJL_ERR_DEVICE;
  return dev == sk->device ? QJL_OK : QJL_ERR_INVALID_ARGUMENT;
}

qjl_status from_hip(hipError_t e) { return e == hipSuccess ? QJL_OK : QJL_ERR_DEVICE; }

}  // namespace

extern "C" {

const char *qjl_status_string(qjl_status s) {
  switch (s) {
    case QJL_OK: return "QJL_OK";
    case QJL_ERR_INVALID_ARGUMENT: return "QJL_ERR_INVALID_ARGUMENT";
    case QJL_ERR_UNSUPPORTED: return "QJL_ERR_UNSUPPORTED";
    case QJL_ERR_OUT_OF_MEMORY: return "QJL_ERR_OUT_OF_MEMORY";
    case QJL_ERR_DEVICE: return "QJL_ERR_DEVICE";
    default: break;
  }
  return "QJL_ERR_UNKNOWN";
}

const char *qjl_version(void) { return "qjl 0.1.0 gfx950"; }

qjl_status qjl_generate_sketch_host(uint64_t seed, int32_t d, int32_t m, int32_t variant,
                                    float *S_f32, uint16_t *S_bf16, int8_t *D_signs,
                                    int32_t *perm, float *G, float *dither_mag) {
  qjl_status st = validate_sketch_params(d, m, variant, 0.f, /*check_rho=*/false);
  if (st != QJL_OK) return st;
  HostSketch hs;
  hs.seed = seed;
  hs.d = d;
  hs.m = m;
  hs.variant = variant;
  try {
    generate_host_sketch(hs);
  } catch (const std::bad_alloc &) {
    return QJL_ERR_OUT_OF_MEMORY;
  }
  const size_t md = (size_t)m * d;
  if (variant == QJL_VARIANT_DENSE) {
    if (S_f32) std::memcpy(S_f32, hs.S32.data(), md * sizeof(float));
    if (S_bf16) std::memcpy(S_bf16, hs.S16.data(), md * sizeof(uint16_t));
  } else {
    if (D_signs) std::memcpy(D_signs, hs.D.data(), hs.D.size());
    if (perm) std::memcpy(perm, hs.P.data(), hs.P.size() * sizeof(int32_t));
    if (G) std::memcpy(G, hs.G.data(), hs.G.size() * sizeof(float));
  }
  if (dither_mag) std::memcpy(dither_mag, hs.Dmag.data(), (size_t)m * sizeof(float));
  return QJL_OK;
}

qjl_status qjl_make_sketch(uint64_t seed, int32_t d, int32_t m, int32_t variant, float rho,
                           qjl_sketch **out) {
  if (!out) return QJL_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  qjl_status st = validate_sketch_params(d, m, variant, rho);
  if (st != QJL_OK) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return QJL_ERR_DEVICE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return QJL_ERR_DEVICE;

  qjl_sketch *sk = new (std::nothrow) qjl_sketch;
  if (!sk) return QJL_ERR_OUT_OF_MEMORY;
  sk->device = dev;
  HostSketch &hs = sk->host;
  hs.seed = seed;
  hs.d = d;
  hs.m = m;
  hs.variant = variant;
  hs.rho = rho;
  sk->dither_key = stream_key(seed, STREAM_DITHER_SIGN);
  try {
    generate_host_sketch(hs);
  } catch (const std::bad_alloc &) {
    delete sk;
    return QJL_ERR_OUT_OF_MEMORY;
  }

  // Lay out every device array in one allocation.
  const size_t md = (size_t)m * d;
  std::vector<unsigned char> blob;
  size_t off_a = 0, off_b = 0, off_c = 0, off_d = 0, off_e = 0, off_f = 0, total = 0;
  try {
    if (variant == QJL_VARIANT_DENSE) {
      off_a = 0;                                             // S32   float[md]
      off_b = round_up(off_a + md * 4, 256);                 // S16f  float[md]
      off_c = round_up(off_b + md * 4, 256);                 // S16mfma u16[md]
      off_d = round_up(off_c + md * 2, 256);                 // S32T  float[md]
      off_e = round_up(off_d + md * 4, 256);                 // S16fT float[md]
      off_f = round_up(off_e + md * 4, 256);                 // Dmag  float[m]
      total = round_up(off_f + (size_t)m * 4, 256);
      blob.assign(total, 0);
      std::memcpy(blob.data() + off_a, hs.S32.data(), md * 4);
      float *s16f = reinterpret_cast<float *>(blob.data() + off_b);
      float *s32t = reinterpret_cast<float *>(blob.data() + off_d);
      float *s16ft = reinterpret_cast<float *>(blob.data() + off_e);
      for (size_t i = 0; i < md; ++i) {
        const uint32_t u = (uint32_t)hs.S16[i] << 16;
        std::memcpy(&s16f[i], &u, 4);
      }
      for (int j = 0; j < m; ++j)
        for (int c = 0; c < d; ++c) {
          s32t[(size_t)c * m + j] = hs.S32[(size_t)j * d + c];
          s16ft[(size_t)c * m + j] = s16f[(size_t)j * d + c];
        }
      build_mfma_b_layout(hs.S16.data(), d, m, reinterpret_cast<uint16_t *>(blob.data() + off_c));
    } else {
      const size_t nbd = (size_t)(m / d) * d;
      off_a = 0;                                  // Dsign u32[nbd]
      off_b = round_up(off_a + nbd * 4, 256);     // P     i32[nbd]
      off_c = round_up(off_b + nbd * 4, 256);     // Gs    f32[nbd]
      off_d = round_up(off_c + nbd * 4, 256);     // Fmfma u16[md] (matrix-core first stage)
      off_f = round_up(off_d + (fqjl_mfma_image_shape(d, m) ? md * 2 : 0), 256);  // Dmag f32[m]
      total = round_up(off_f + (size_t)m * 4, 256);
      blob.assign(total, 0);
      if (fqjl_mfma_image_shape(d, m))
        build_fqjl_mfma_image(hs, reinterpret_cast<uint16_t *>(blob.data() + off_d));
      uint32_t *ds = reinterpret_cast<uint32_t *>(blob.data() + off_a);
      float *gs = reinterpret_cast<float *>(blob.data() + off_c);
      const float inv = (float)(1.0 / std::sqrt((double)d));
      for (size_t i = 0; i < nbd; ++i) {
        ds[i] = hs.D[i] < 0 ? 0x80000000u : 0u;
        gs[i] = hs.G[i] * inv;
      }
      std::memcpy(blob.data() + off_b, hs.P.data(), nbd * 4);
    }
    std::memcpy(blob.data() + off_f, hs.Dmag.data(), (size_t)m * 4);
  } catch (const std::bad_alloc &) {
    delete sk;
    return QJL_ERR_OUT_OF_MEMORY;
  }
  if (hipMalloc(&sk->dmem, total) != hipSuccess) {
    (void)hipGetLastError();
    delete sk;
    return QJL_ERR_OUT_OF_MEMORY;
  }
  if (hipMemcpy(sk->dmem, blob.data(), total, hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(sk->dmem);
    delete sk;
    return QJL_ERR_DEVICE;
  }
  unsigned char *base = static_cast<unsigned char *>(sk->dmem);
  if (variant == QJL_VARIANT_DENSE) {
    sk->S32 = reinterpret_cast<const float *>(base + off_a);
    sk->S16f = reinterpret_cast<const float *>(base + off_b);
    sk->S16mfma = reinterpret_cast<const uint16_t *>(base + off_c);
    sk->S32T = reinterpret_cast<const float *>(base + off_d);
    sk->S16fT = reinterpret_cast<const float *>(base + off_e);
  } else {
    sk->Dsign = reinterpret_cast<const uint32_t *>(base + off_a);
    sk->P = reinterpret_cast<const int32_t *>(base + off_b);
    sk->Gs = reinterpret_cast<const float *>(base + off_c);
    if (fqjl_mfma_image_shape(d, m)) sk->Fmfma = reinterpret_cast<const uint16_t *>(base + off_d);
  }
  sk->Dmag = reinterpret_cast<const float *>(base + off_f);
  *out = sk;
  return QJL_OK;
}

qjl_status qjl_destroy_sketch(qjl_sketch *sk) {
  if (!sk) return QJL_ERR_INVALID_ARGUMENT;
  qjl_status st = QJL_OK;
  if (sk->dmem) {
    int prev = -1;
    (void)hipGetDevice(&prev);
    if (prev != sk->device) (void)hipSetDevice(sk->device);
    if (hipFree(sk->dmem) != hipSuccess) st = QJL_ERR_DEVICE;
    if (prev >= 0 && prev != sk->device) (void)hipSetDevice(prev);
  }
  delete sk;
  return st;
}

qjl_status qjl_sketch_info(const qjl_sketch *sk, uint64_t *seed, int32_t *d, int32_t *m,
                           int32_t *variant, float *rho, int32_t *device) {
  if (!sk) return QJL_ERR_INVALID_ARGUMENT;
  if (seed) *seed = sk->host.seed;
  if (d) *d = sk->host.d;
  if (m) *m = sk->host.m;
  if (variant) *variant = sk->host.variant;
  if (rho) *rho = sk->host.rho;
  if (device) *device = sk->device;
  return QJL_OK;
}

qjl_status qjl_sketch_export(const qjl_sketch *sk, float *S_f32, uint16_t *S_bf16) {
  if (!sk) return QJL_ERR_INVALID_ARGUMENT;
  const HostSketch &hs = sk->host;
  const size_t md = (size_t)hs.m * hs.d;
  if (hs.variant == QJL_VARIANT_DENSE) {
    if (S_f32) std::memcpy(S_f32, hs.S32.data(), md * 4);
    if (S_bf16) std::memcpy(S_bf16, hs.S16.data(), md * 2);
    return QJL_OK;
  }
  if (S_bf16) return QJL_ERR_INVALID_ARGUMENT;
  if (S_f32) {
    std::vector<double> ex;
    try {
      fqjl_explicit(hs, ex);
    } catch (const std::bad_alloc &) {
      return QJL_ERR_OUT_OF_MEMORY;
    }
    for (size_t i = 0; i < md; ++i) S_f32[i] = (float)ex[i];
  }
  return QJL_OK;
}

namespace {

// Shared by qjl_quantize_keys and qjl_quantize_keys_into, after their own
// argument checks: the device check and the kernel dispatch.
qjl_status quantize_dispatch(const qjl_sketch *sk, const void *K, int32_t dtype, int64_t n,
                             int64_t key_index_base, const RowMap &map, float *norms,
                             uint32_t *bits, void *stream) {
  qjl_status st = check_device(sk);
  if (st != QJL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sk->host.variant != QJL_VARIANT_DENSE)
    return from_hip(launch_fqjl(sk, K, dtype, n, key_index_base, map, norms, bits, nullptr, s));
  if (quantize_mfma_supported(sk, K, dtype, bits))
    return from_hip(launch_quantize_mfma(sk, K, n, map, norms, bits, s));
  return from_hip(launch_quantize_generic(sk, K, dtype, n, key_index_base, map, norms, bits, s));
}

}  // namespace

qjl_status qjl_quantize_keys(const qjl_sketch *sk, const void *K, int32_t dtype, int64_t n_keys,
                             int64_t key_index_base, float *norms_out, uint32_t *bits_out,
                             void *stream) {
  if (!sk || n_keys < 0 || key_index_base < 0) return QJL_ERR_INVALID_ARGUMENT;
  if (dtype != QJL_DTYPE_F32 && dtype != QJL_DTYPE_BF16) return QJL_ERR_INVALID_ARGUMENT;
  if (n_keys == 0) return QJL_OK;
  if (!K || !norms_out || !bits_out) return QJL_ERR_INVALID_ARGUMENT;
  const uintptr_t esz = dtype == QJL_DTYPE_F32 ? 4 : 2;
  if (!aligned(K, esz) || !aligned(norms_out, 4) || !aligned(bits_out, 4))
    return QJL_ERR_INVALID_ARGUMENT;
  return quantize_dispatch(sk, K, dtype, n_keys, key_index_base, RowMap{}, norms_out, bits_out,
                           stream);
}

qjl_status qjl_quantize_keys_into(const qjl_sketch *sk, const void *K, int32_t dtype,
                                  int64_t n_groups, int64_t keys_per_group,
                                  int64_t cache_rows_per_group, int64_t first_row,
                                  int64_t key_index_base, float *norms_cache,
                                  uint32_t *bits_cache, void *stream) {
  if (!sk || n_groups < 0 || keys_per_group < 0 || cache_rows_per_group < 0 || first_row < 0 ||
      key_index_base < 0)
    return QJL_ERR_INVALID_ARGUMENT;
  if (dtype != QJL_DTYPE_F32 && dtype != QJL_DTYPE_BF16) return QJL_ERR_INVALID_ARGUMENT;
  // the new rows must lie inside each group's slice of the cache
  if (first_row > cache_rows_per_group || keys_per_group > cache_rows_per_group - first_row)
    return QJL_ERR_INVALID_ARGUMENT;
  if (n_groups == 0 || keys_per_group == 0) return QJL_OK;
  const int64_t big = INT64_MAX / 2;
  if (n_groups > big / keys_per_group || n_groups > big / cache_rows_per_group)
    return QJL_ERR_INVALID_ARGUMENT;  // key or cache row counts overflow
  const int64_t n = n_groups * keys_per_group;
  if (n >= ((int64_t)1 << 32)) return QJL_ERR_UNSUPPORTED;  // rows are mapped in 32 bits
  if (!K || !norms_cache || !bits_cache) return QJL_ERR_INVALID_ARGUMENT;
  const uintptr_t esz = dtype == QJL_DTYPE_F32 ? 4 : 2;
  if (!aligned(K, esz) || !aligned(norms_cache, 4) || !aligned(bits_cache, 4))
    return QJL_ERR_INVALID_ARGUMENT;
  RowMap map;
  map.per_group = keys_per_group;
  map.stride = cache_rows_per_group;
  map.first = first_row;
  return quantize_dispatch(sk, K, dtype, n, key_index_base, map, norms_cache, bits_cache, stream);
}

qjl_status qjl_project_query(const qjl_sketch *sk, const void *q, int32_t dtype,
                             int64_t n_queries, float *Sq_out, void *stream) {
  if (!sk || n_queries < 0) return QJL_ERR_INVALID_ARGUMENT;
  if (dtype != QJL_DTYPE_F32 && dtype != QJL_DTYPE_BF16) return QJL_ERR_INVALID_ARGUMENT;
  if (n_queries == 0) return QJL_OK;
  if (!q || !Sq_out) return QJL_ERR_INVALID_ARGUMENT;
  const uintptr_t esz = dtype == QJL_DTYPE_F32 ? 4 : 2;
  if (!aligned(q, esz) || !aligned(Sq_out, 4)) return QJL_ERR_INVALID_ARGUMENT;
  qjl_status st = check_device(sk);
  if (st != QJL_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sk->host.variant != QJL_VARIANT_DENSE) {
    if (fqjl_project_mfma_supported(sk, q, dtype, Sq_out))
      return from_hip(launch_fqjl_project_mfma(sk, q, n_queries, Sq_out, s));
    return from_hip(launch_fqjl(sk, q, dtype, n_queries, 0, RowMap{}, nullptr, nullptr, Sq_out, s));
  }
  if (project_mfma_supported(sk, q, dtype, n_queries, Sq_out))
    return from_hip(launch_project_mfma(sk, q, n_queries, Sq_out, s));
  return from_hip(launch_project_dense(sk, q, dtype, n_queries, Sq_out, s));
}

qjl_status qjl_score(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                     const float *norms, int64_t n_groups, int64_t n_q_per_group,
                     int64_t n_k_per_group, float *scores_out, void *stream) {
  if (!sk || n_groups < 0 || n_q_per_group < 0 || n_k_per_group < 0)
    return QJL_ERR_INVALID_ARGUMENT;
  if (n_groups == 0 || n_q_per_group == 0 || n_k_per_group == 0) return QJL_OK;
  if (!Sq || !bits || !norms || !scores_out) return QJL_ERR_INVALID_ARGUMENT;
  if (!aligned(Sq, 4) || !aligned(bits, 4) || !aligned(norms, 4) || !aligned(scores_out, 4))
    return QJL_ERR_INVALID_ARGUMENT;
  qjl_status st = check_device(sk);
  if (st != QJL_OK) return st;
  return from_hip(launch_score(sk, Sq, bits, norms, n_groups, n_q_per_group, n_k_per_group,
                               scores_out, static_cast<hipStream_t>(stream)));
}

qjl_status qjl_decode_attention_workspace_size(const qjl_sketch *sk, int64_t n_groups,
                                               int64_t n_q_per_group, int64_t n_k_per_group,
                                               int32_t d_v, size_t *bytes_out) {
  if (!sk || !bytes_out || n_groups < 0 || n_q_per_group < 0 || n_k_per_group < 0 || d_v < 1)
    return QJL_ERR_INVALID_ARGUMENT;
  if (n_groups == 0 || n_q_per_group == 0 || n_k_per_group == 0) {
    *bytes_out = 0;
    return QJL_OK;
  }
  qjl_status st = check_device(sk);
  if (st != QJL_OK) return st;
  *bytes_out = attention_workspace_bytes(sk, n_groups, n_q_per_group, n_k_per_group, d_v);
  return QJL_OK;
}

qjl_status qjl_decode_attention(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                                int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                                float softmax_scale, void *workspace, size_t workspace_bytes,
                                float *out, void *stream) {
  bool noop = false;
  qjl_status st = attention_check_args(sk, Sq, bits, norms, V, v_dtype, d_v, n_groups,
                                       n_q_per_group, n_k_per_group, softmax_scale, out, &noop);
  if (st != QJL_OK || noop) return st;
  if (!workspace || !aligned(workspace, 16)) return QJL_ERR_INVALID_ARGUMENT;
  if (workspace_bytes <
      attention_workspace_bytes(sk, n_groups, n_q_per_group, n_k_per_group, d_v))
    return QJL_ERR_INVALID_ARGUMENT;
  return attention_run(sk, Sq, bits, norms, V, v_dtype, d_v, n_groups, n_q_per_group,
                       n_k_per_group, softmax_scale, static_cast<float *>(workspace), out,
                       stream);
}

}  // extern "C"

namespace qjl {

qjl_status attention_check_args(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                                const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                                int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                                float softmax_scale, const float *out, bool *noop) {
  *noop = false;
  if (!sk || n_groups < 0 || n_q_per_group < 0 || n_k_per_group < 0 || d_v < 1)
    return QJL_ERR_INVALID_ARGUMENT;
  if (v_dtype != QJL_DTYPE_F32 && v_dtype != QJL_DTYPE_BF16) return QJL_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(softmax_scale)) return QJL_ERR_INVALID_ARGUMENT;
  if (n_groups == 0 || n_q_per_group == 0) {
    *noop = true;
    return QJL_OK;
  }
  if (n_k_per_group == 0) return QJL_ERR_INVALID_ARGUMENT;  // softmax over no keys
  if (!Sq || !bits || !norms || !V || !out) return QJL_ERR_INVALID_ARGUMENT;
  const size_t vsz = v_dtype == QJL_DTYPE_F32 ? 4 : 2;
  if (!aligned(Sq, 4) || !aligned(bits, 4) || !aligned(norms, 4) || !aligned(V, vsz) ||
      !aligned(out, 4))
    return QJL_ERR_INVALID_ARGUMENT;
  return check_device(sk);
}

qjl_status attention_run(const qjl_sketch *sk, const float *Sq, const uint32_t *bits,
                         const float *norms, const void *V, int32_t v_dtype, int32_t d_v,
                         int64_t n_groups, int64_t n_q_per_group, int64_t n_k_per_group,
                         float softmax_scale, float *ws, float *out, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (attention_fused_supported(sk, bits, V, v_dtype, d_v, n_k_per_group))
    return from_hip(launch_attention_fused(sk, Sq, bits, norms, V, n_groups, n_q_per_group,
                                           n_k_per_group, softmax_scale, ws, out, s));
  hipError_t e = launch_score(sk, Sq, bits, norms, n_groups, n_q_per_group, n_k_per_group, ws, s);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(launch_attention_softmax(ws, V, v_dtype, d_v, n_groups, n_q_per_group,
                                           n_k_per_group, softmax_scale, out, s));
}

float estimator_scale(int m, float rho) {
  const double c = std::sqrt(M_PI / 2.0) * std::sqrt(1.0 + (double)rho * (double)rho) / (double)m;
  return (float)c;
}
}  // namespace qjl
