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
diagonal G, 4 dither.  The dither stream draws one word per two coordinate
pairs (see ``dither_pairs``): each 32-bit half gives a 20-bit radius uniform
and one of 4096 equally spaced angles, both exact in fp32 and fp64 alike.
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
STREAM_DITHER = 4


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


def dither_pairs(seed: int, key_index: np.ndarray, m: int) -> np.ndarray:
    """Dither noise xi[i, j] for global key indices ``key_index`` and j < m.

    Key i draws m/4 words h_w = r(seed, 4, i*(m/4) + w), w < m/4; word w
    serves coordinate pairs p = 2w (its high 32 bits) and p = 2w + 1 (its low
    32 bits).  From a 32-bit half v: a = v >> 12 (20 bits), k = v & 0xFFF, and

        u1 = (a + 1) * 2**-20  in (0, 1],   R = sqrt(-2 ln u1)
        theta = 2 pi (k + 1/2) / 4096
        xi[i, 2p] = R cos(theta),   xi[i, 2p+1] = R sin(theta)

    Box-Muller (1958) with the angle on 4096 equally spaced values, offset by
    half a step so that no angle has a zero cosine or sine.  The radius is
    Rayleigh as in the continuous method (its top 2**-20 of tail mass cut),
    and since the average of exp(i n theta) over the angles vanishes for
    0 < |n| < 4096, every joint moment of (xi_2p, xi_2p+1) of total order
    below 4096 equals that of two independent standard normals.
    """
    key_index = np.asarray(key_index, dtype=np.uint64).reshape(-1)
    if m % 4:
        raise ValueError("the dither draws one word per two coordinate pairs: m % 4 == 0")
    words = m // 4
    ctr = key_index[:, None] * np.uint64(words) + np.arange(words, dtype=np.uint64)[None, :]
    h = draw(seed, STREAM_DITHER, ctr)
    halves = np.empty((key_index.shape[0], 2 * words), dtype=np.uint64)
    halves[:, 0::2] = h >> np.uint64(32)                    # pair 2w
    halves[:, 1::2] = h & np.uint64(0xFFFFFFFF)             # pair 2w + 1
    a = (halves >> np.uint64(12)).astype(np.float64)
    k = (halves & np.uint64(0xFFF)).astype(np.float64)
    u1 = (a + 1.0) * 2.0 ** -20
    rad = np.sqrt(-2.0 * np.log(u1))
    th = TWO_PI * (k + 0.5) / 4096.0
    out = np.empty((key_index.shape[0], m), dtype=np.float64)
    out[:, 0::2] = rad * np.cos(th)
    out[:, 1::2] = rad * np.sin(th)
    return out
