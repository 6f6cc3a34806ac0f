// The bf16 operand image of a dense sketch for v_mfma_f32_32x32x16_bf16,
// shared by the key quantizer and the query projection (both contract rows
// of S with bf16 vectors loaded the same way, so they apply the same sums).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qjl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

// The 16-byte chunk (8 bf16 values) of a vector that lane half h feeds to
// MFMA step t: the two lanes of a vector read adjacent chunks in the same
// load instruction, so one instruction covers 32 contiguous bytes of each of
// its 32 rows.
__host__ __device__ constexpr int qm_chunk(int h, int t) { return 2 * t + h; }

// Host: write S (bf16 bits, m x d row-major) in the operand order.  Tile
// tau = 2 p + s (p < W/2 word pairs, s < 2, W = m/32): row r = 8 a + 4 h + b
// of the tile is coordinate 32 (p + h W/2) + 16 s + 4 a + b; for tile tau,
// step t and lane l = r + 32 hh the 8 values S[row][8 qm_chunk(hh, t) + e],
// e < 8, are contiguous.  Needs d % 16 == 0 and m % 64 == 0 (otherwise the
// image is left unwritten and unused).
void build_mfma_b_layout(const uint16_t *S16, int d, int m, uint16_t *out);

}  // namespace qjl
