// Host-side generation of the random sketch parameters.
//
// Dense S (QJL abstract, Majid Daliri's scholarfeed page: a JL transform;
// "Fast Quantized Johnson-Lindenstrauss Transforms" page: a dense Gaussian
// projection): S[j][c] = N(j d + c) on stream 0, rounded to float32, and the
// bfloat16 rounding of that float32 value for bfloat16 inputs.
//
// FQJL blocks (same page: randomized Hadamard transforms with a Gaussian
// second diagonal and a uniform random permutation between them): per block
// b < m/d, D_b[c] = +1 if the top bit of r(seed, 1, b d + c) is 0 else -1;
// P_b by Fisher-Yates with t = floor(U(b d + i) (i + 1)) on stream 2;
// G_b[c] = float32(N(b d + c)) on stream 3.
//
// Dither magnitudes (same page, Key concepts: D-FQJL's Gaussian dither), for
// every variant: a_j = float32(|N(j)|), j < m, on stream 4; each key's signs
// are drawn on the device (device_common.h).
//
// U(i) = ((r >> 11) + 0.5) 2^-53 and N(i) = sqrt(-2 ln U(2i)) cos(2 pi U(2i+1))
// (Box-Muller), evaluated in double with the C library's log and cos.
#include <cmath>
#include <cstring>

#include "qjl_internal.h"

namespace qjl {

static const double TWO_PI = 6.283185307179586;  // nearest double to 2 pi

static inline double uniform53(uint64_t r) {
  return ((double)(r >> 11) + 0.5) * 0x1p-53;
}

static inline double gaussian(uint64_t key, uint64_t i) {
  const double ua = uniform53(stream_draw(key, 2 * i));
  const double ub = uniform53(stream_draw(key, 2 * i + 1));
  return std::sqrt(-2.0 * std::log(ua)) * std::cos(TWO_PI * ub);
}

uint16_t f32_to_bf16_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

qjl_status validate_sketch_params(int32_t d, int32_t m, int32_t variant, float rho,
                                  bool check_rho) {
  if (variant < QJL_VARIANT_DENSE || variant > QJL_VARIANT_PFQJL) return QJL_ERR_INVALID_ARGUMENT;
  if (m < 32 || m % 32 != 0) return QJL_ERR_INVALID_ARGUMENT;
  if (d < 1) return QJL_ERR_INVALID_ARGUMENT;
  if (check_rho) {
    if (!(rho >= 0.f) || !std::isfinite(rho)) return QJL_ERR_INVALID_ARGUMENT;
    // D-FQJL is the dithered construction, P-FQJL the undithered one
    if (variant == QJL_VARIANT_DFQJL && !(rho > 0.f)) return QJL_ERR_INVALID_ARGUMENT;
    if (variant == QJL_VARIANT_PFQJL && rho != 0.f) return QJL_ERR_INVALID_ARGUMENT;
  }
  if (m > QJL_MAX_M) return QJL_ERR_UNSUPPORTED;
  if (variant == QJL_VARIANT_DENSE) {
    if (d > QJL_MAX_D) return QJL_ERR_UNSUPPORTED;
  } else {
    if (!is_pow2(d) || d < 8 || d > 256 || m % d != 0) return QJL_ERR_UNSUPPORTED;
  }
  return QJL_OK;
}

void generate_host_sketch(HostSketch &hs) {
  const int d = hs.d, m = hs.m;
  {
    const uint64_t key = stream_key(hs.seed, STREAM_DITHER);
    hs.Dmag.resize((size_t)m);
    for (int j = 0; j < m; ++j) hs.Dmag[(size_t)j] = (float)std::fabs(gaussian(key, (uint64_t)j));
  }
  if (hs.variant == QJL_VARIANT_DENSE) {
    const uint64_t key = stream_key(hs.seed, STREAM_DENSE);
    hs.S32.resize((size_t)m * d);
    hs.S16.resize((size_t)m * d);
    for (size_t i = 0; i < (size_t)m * d; ++i) {
      const float s = (float)gaussian(key, i);
      hs.S32[i] = s;
      hs.S16[i] = f32_to_bf16_rne(s);
    }
    return;
  }
  const int nb = m / d;
  hs.D.resize((size_t)nb * d);
  hs.P.resize((size_t)nb * d);
  hs.G.resize((size_t)nb * d);
  const uint64_t kd = stream_key(hs.seed, STREAM_D);
  const uint64_t kp = stream_key(hs.seed, STREAM_P);
  const uint64_t kg = stream_key(hs.seed, STREAM_G);
  for (int b = 0; b < nb; ++b) {
    int8_t *D = &hs.D[(size_t)b * d];
    int32_t *P = &hs.P[(size_t)b * d];
    float *G = &hs.G[(size_t)b * d];
    for (int c = 0; c < d; ++c) {
      D[c] = (stream_draw(kd, (uint64_t)b * d + c) >> 63) ? -1 : 1;
      P[c] = c;
      G[c] = (float)gaussian(kg, (uint64_t)b * d + c);
    }
    if (hs.variant == QJL_VARIANT_DFQJL) continue;  // no permutation: P_b = I
    for (int i = d - 1; i >= 1; --i) {
      const double u = uniform53(stream_draw(kp, (uint64_t)b * d + i));
      const int t = (int)std::floor(u * (double)(i + 1));
      const int32_t tmp = P[i];
      P[i] = P[t];
      P[t] = tmp;
    }
  }
}

// In-place unnormalised Walsh-Hadamard transform (natural order) in double.
static void fwht_d(double *x, int d) {
  for (int h = 1; h < d; h *= 2)
    for (int i = 0; i < d; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        const double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

void fqjl_explicit(const HostSketch &hs, std::vector<double> &out) {
  const int d = hs.d, m = hs.m, nb = m / d;
  out.assign((size_t)m * d, 0.0);
  std::vector<double> u(d), v(d);
  const double inv = 1.0 / std::sqrt((double)d);
  for (int b = 0; b < nb; ++b)
    for (int c = 0; c < d; ++c) {
      for (int i = 0; i < d; ++i) u[i] = 0.0;
      u[c] = (double)hs.D[(size_t)b * d + c];
      fwht_d(u.data(), d);
      for (int i = 0; i < d; ++i) u[i] *= inv;
      for (int i = 0; i < d; ++i)
        v[i] = u[hs.P[(size_t)b * d + i]] * (double)hs.G[(size_t)b * d + i];
      fwht_d(v.data(), d);
      for (int i = 0; i < d; ++i) out[((size_t)b * d + i) * d + c] = v[i];
    }
}

}  // namespace qjl
