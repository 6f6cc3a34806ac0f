// Host-side operand images of the matrix-core kernels, written once per
// sketch by qjl_make_sketch: the dense S in the MFMA operand order of
// mfma_image.h, and the +-1 first stage of the FQJL blocks.  Plain host code
// (no kernels), so it also builds and runs under the CPU sanitizers.
#include "mfma_image.h"
#include "qjl_internal.h"

namespace qjl {

// Host: write S in the operand order of mfma_image.h.
void build_mfma_b_layout(const uint16_t *S16, int d, int m, uint16_t *out) {
  if (d % 16 != 0 || m % 64 != 0) return;  // the MFMA path's shapes; image unused otherwise
  const int T = d / 16, W = m / 32;
  for (int tau = 0; tau < m / 32; ++tau) {
    const int p = tau >> 1, s = tau & 1;
    for (int t = 0; t < T; ++t)
      for (int l = 0; l < 64; ++l) {
        const int r = l & 31, hh = l >> 5;
        const int a = r >> 3, h = (r >> 2) & 1, b = r & 3;
        const int j = 32 * (p + h * (W / 2)) + 16 * s + 4 * a + b;
        for (int e = 0; e < 8; ++e)
          out[(((size_t)tau * T + t) * 64 + l) * 8 + e] =
              S16[(size_t)j * d + 8 * qm_chunk(hh, t) + e];
      }
  }
}

bool fqjl_mfma_image_shape(int d, int m) {
  return d == 128 && (m == 128 || m == 256 || m == 512);
}

// Host: operand image of the blocks' first stage M_b = Pi_b H diag(D_b),
// with row i negated where G_b[i] < 0 (the kernel then scales by |G_b[i]|).
void build_fqjl_mfma_image(const HostSketch &hs, uint16_t *out) {
  const int d = hs.d, m = hs.m;
  if (!fqjl_mfma_image_shape(d, m)) return;
  const int T = d / 16, NB = m / d;
  for (int b = 0; b < NB; ++b)
    for (int p = 0; p < 4; ++p) {
      const int tau = 4 * b + p;
      for (int t = 0; t < T; ++t)
        for (int l = 0; l < 64; ++l) {
          const int r = l & 31, hh = l >> 5;
          const int a = r >> 3, h = (r >> 2) & 1, bb = r & 3;
          const int i = 64 * h + 16 * p + 4 * a + bb;  // coordinate of block b
          const int pi = hs.P[(size_t)b * d + i];      // row of H it takes
          const int gneg = hs.G[(size_t)b * d + i] < 0.f ? 1 : 0;  // sign of G_b[i], see below
          for (int e = 0; e < 8; ++e) {
            const int c = 8 * qm_chunk(hh, t) + e;
            const int neg = (__builtin_popcount((unsigned)(pi & c)) & 1) ^
                            (hs.D[(size_t)b * d + c] < 0 ? 1 : 0) ^ gneg;
            out[(((size_t)tau * T + t) * 64 + l) * 8 + e] = neg ? 0xBF80 : 0x3F80;  // -1, +1
          }
        }
    }
}

}  // namespace qjl
