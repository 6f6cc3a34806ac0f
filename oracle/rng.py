"""Counter-based random streams for the oracle (plain numpy, uint64).

Test infrastructure only: nothing in the product path imports this module.

The pages fix no random number generator, so the sketch is defined by this
one.  It is built on the SplitMix64 output function of Steele, Lea and Flood
("Fast splittable pseudorandom number generators", OOPSLA 2014), written
here from that published definition:

    mix64(z): z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
              z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31

with all arithmetic mod 2**64 and PHI = 0x9E3779B97F4A7C15.

    key(seed, stream)   = mix64(seed + PHI * (stream + 1))
    r(seed, stream, i)  = mix64(key(seed, stream) + PHI * (i + 1))

so r(seed, stream, 0), r(seed, stream, 1), ... is exactly the SplitMix64
sequence started from state key(seed, stream).

Derived variates (all in float64 unless stated):

    U(i)  = ((r >> 11) + 0.5) * 2**-53                      in (0, 1)
    N(i)  = sqrt(-2 ln U(2i)) * cos(2 pi U(2i+1))           (Box and Muller, 1958)

Streams: 0 dense S, 1 Rademacher diagonal D, 2 permutation P, 3 Gaussian
diagonal G, 4 dither magnitudes, 5 dither signs.  A sketch with dither holds
m Gaussian magnitudes |N(j)| (stream 4, drawn once with the sketch, like G);
each key draws its own m random signs from stream 5, one 64-bit word per 64
coordinates (see ``dither_signs``), so the dither of any one key is m
independent N(0, 1) values, independent of the transform.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
PHI = 0x9E3779B97F4A7C15
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)
TWO_PI = 6.283185307179586  # the float64 nearest 2*pi, used verbatim on both sides

STREAM_DENSE = 0
STREAM_D = 1
STREAM_P = 2
STREAM_G = 3
STREAM_DITHER = 4       # the sketch's dither magnitudes
STREAM_DITHER_SIGN = 5  # each key's dither signs


def mix64(z) -> np.ndarray:
    """SplitMix64 finaliser on a uint64 array (wrapping multiply)."""
    z = np.asarray(z, dtype=np.uint64).copy()
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= _C1
        z ^= z >> np.uint64(27)
        z *= _C2
        z ^= z >> np.uint64(31)
    return z


def mix64_int(z: int) -> int:
    """The same finaliser on a Python int (used for scalar keys)."""
    z &= MASK64
    z ^= z >> 30
    z = (z * 0xBF58476D1CE4E5B9) & MASK64
    z ^= z >> 27
    z = (z * 0x94D049BB133111EB) & MASK64
    z ^= z >> 31
    return z


def stream_key(seed: int, stream: int) -> int:
    return mix64_int((seed + PHI * (stream + 1)) & MASK64)


def draw(seed: int, stream: int, idx) -> np.ndarray:
    """r(seed, stream, i) for an array of counters i (uint64)."""
    key = np.uint64(stream_key(seed, stream))
    i = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + np.uint64(PHI) * (i + np.uint64(1))
    return mix64(z)


def uniform53(r: np.ndarray) -> np.ndarray:
    """((r >> 11) + 0.5) * 2**-53: exact in float64, strictly inside (0, 1)."""
    return ((r >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53


def gaussian_exact(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """N(offset), ..., N(offset+count-1) with the C library's log/cos.

    Evaluated one value at a time through ``math.log`` / ``math.cos`` so the
    result is bit-for-bit what any C program calling the same libm computes
    for the same float64 arguments.
    """
    idx = np.arange(offset, offset + count, dtype=np.uint64)
    u_a = uniform53(draw(seed, stream, 2 * idx))
    u_b = uniform53(draw(seed, stream, 2 * idx + 1))
    out = np.empty(count, dtype=np.float64)
    log, cos, sqrt = math.log, math.cos, math.sqrt
    for t in range(count):
        out[t] = sqrt(-2.0 * log(float(u_a[t]))) * cos(TWO_PI * float(u_b[t]))
    return out


def gaussian_fast(seed: int, stream: int, idx) -> np.ndarray:
    """N(i) vectorised with numpy's log/cos (may differ from libm by an ulp)."""
    idx = np.asarray(idx, dtype=np.uint64)
    u_a = uniform53(draw(seed, stream, np.uint64(2) * idx))
    u_b = uniform53(draw(seed, stream, np.uint64(2) * idx + np.uint64(1)))
    return np.sqrt(-2.0 * np.log(u_a)) * np.cos(TWO_PI * u_b)


def dither_magnitudes(seed: int, m: int, exact: bool = True) -> np.ndarray:
    """The sketch's dither magnitudes a[j] = |N(j)|, j < m, on stream 4,
    rounded to float32 (returned as float64): drawn once per sketch, as the
    Gaussian diagonal G is, and held in float32 on both sides."""
    g = (gaussian_exact(seed, STREAM_DITHER, m) if exact
         else gaussian_fast(seed, STREAM_DITHER, np.arange(m)))
    return np.abs(g).astype(np.float32).astype(np.float64)


def dither_signs(seed: int, key_index: np.ndarray, m: int) -> np.ndarray:
    """Dither signs s[i, j] in {+1, -1} for global key indices ``key_index``
    and coordinates j < m.

    Key i draws W = ceil(m / 64) words h_w = r(seed, 5, i*W + w).  The 32-bit
    sign word v (coordinates 32v .. 32v + 31) is the high half of h_{v//2}
    for even v and its low half for odd v; bit j % 32 of word j // 32
    (least significant first) is 1 for s[i, j] = -1 and 0 for +1.
    """
    key_index = np.asarray(key_index, dtype=np.uint64).reshape(-1)
    words = (m + 63) // 64
    ctr = key_index[:, None] * np.uint64(words) + np.arange(words, dtype=np.uint64)[None, :]
    h = draw(seed, STREAM_DITHER_SIGN, ctr)
    w32 = np.empty((key_index.shape[0], 2 * words), dtype=np.uint64)
    w32[:, 0::2] = h >> np.uint64(32)
    w32[:, 1::2] = h & np.uint64(0xFFFFFFFF)
    j = np.arange(m)
    bit = (w32[:, j // 32] >> (j % 32).astype(np.uint64)[None, :]) & np.uint64(1)
    return np.where(bit == 1, -1.0, 1.0)


def dither(seed: int, key_index: np.ndarray, m: int, magnitudes: np.ndarray) -> np.ndarray:
    """Dither noise xi[i, j] = s[i, j] * a[j]: each key's own random signs on
    the sketch's magnitudes.  For any one key the m values are independent
    N(0, 1) over the sketch's draw (a[j] half-normal, s[i, j] a fair sign
    independent of it), which is all the dithered estimator's unbiasing
    factor sqrt(1 + rho^2) needs; distinct keys get independent signs, so
    their dither vectors are uncorrelated."""
    return dither_signs(seed, key_index, m) * np.asarray(magnitudes, np.float64)[None, :]
