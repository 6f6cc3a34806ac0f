"""The random sketch S (m x d) in float64: dense Gaussian or FQJL blocks.

Test infrastructure only: nothing in the product path imports this module.

Dense: the QJL abstract (scholarfeed page of Majid Daliri, "QJL" abstract)
projects with a Johnson-Lindenstrauss matrix; the Fast Quantized JL page
("Fast Quantized Johnson-Lindenstrauss Transforms", abstract and the
"Title and authors" part of the transcript) names it a dense Gaussian
projection.  S[j, c] ~ N(0, 1) iid.

FQJL: the same page ("The paper" abstract; "Key concepts", P-FQJL) replaces
S by compositions of randomized Hadamard transforms: the diagonal of the
second stage is Gaussian (the first keeps random signs), and a uniform
random permutation sits between the two Hadamard transforms.  One block is

    B_b = H diag(G_b) Pi_b (H / sqrt(d)) diag(D_b)

with Sylvester H (H[i, c] = (-1)^popcount(i & c), entries +-1), D_b
Rademacher, Pi_b the gather (Pi u)_i = u[P_b[i]] and G_b ~ N(0, 1).  m/d
independent blocks are stacked; block b yields coordinates [b d, (b+1) d).
The pages leave the Hadamard normalisation open; with 1/sqrt(d) on the
first transform only, every coordinate of B_b k has variance ||k||^2 over
G, exactly as a dense Gaussian row, so one estimator constant serves both.

The same page names the two constructions the composition combines
("Key concepts"): D-FQJL smooths the sign quantizer with Gaussian dither
and has no permutation (Pi_b = I here), P-FQJL inserts the random
permutation and has no dither.  "fqjl" is the composition with both
(permutation, optional dither); "dfqjl" and "pfqjl" are the two
constructions alone.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import rng


def round_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_f32_to_bf16(x32: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even on the bits).

    bfloat16 keeps the top 16 bits of the float32 pattern.  Written out on the
    integer bits: add 0x7FFF plus the lowest kept bit, then truncate.
    """
    f = np.asarray(x32, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = (u << np.uint64(16)).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def bf16_bits(x_bf16_values: np.ndarray) -> np.ndarray:
    """The uint16 storage pattern of values already representable in bf16."""
    f = np.asarray(x_bf16_values, dtype=np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def sylvester(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix by the doubling recursion [[H, H], [H, -H]]."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform along the last axis.

    Butterfly stages with span 1, 2, 4, ...; equals x @ sylvester(d).T (the
    natural, not sequency, order).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    assert d & (d - 1) == 0
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


@dataclass
class DenseSketch:
    seed: int
    d: int
    m: int
    rho: float
    S64: np.ndarray   # m x d, the Gaussian draws
    S32: np.ndarray   # float32-rounded (as float64)
    S16: np.ndarray   # bfloat16-rounded from S32 (as float64)
    variant: str = "dense"
    dmag: np.ndarray | None = None   # [m] dither magnitudes (rho > 0), float32-rounded

    def effective(self, in_dtype: str) -> np.ndarray:
        """The S actually applied: bf16 inputs use S16, fp32 inputs use S32."""
        return self.S16 if in_dtype == "bf16" else self.S32


@dataclass
class FqjlSketch:
    seed: int
    d: int
    m: int
    rho: float
    D: np.ndarray     # [m/d, d] entries +-1
    P: np.ndarray     # [m/d, d] permutations of range(d)
    G: np.ndarray     # [m/d, d] float32-rounded Gaussians (as float64)
    variant: str = "fqjl"
    dmag: np.ndarray | None = None   # [m] dither magnitudes (rho > 0), float32-rounded

    def explicit(self) -> np.ndarray:
        """The m x d matrix: blocks H diag(G) Pi (H/sqrt d) diag(D) stacked."""
        d = self.d
        H = sylvester(d)
        rows = []
        for b in range(self.m // d):
            Pi = np.zeros((d, d))
            Pi[np.arange(d), self.P[b]] = 1.0          # (Pi u)_i = u[P[i]]
            B = H @ np.diag(self.G[b]) @ Pi @ (H / np.sqrt(d)) @ np.diag(self.D[b])
            rows.append(B)
        return np.vstack(rows)

    def effective(self, in_dtype: str) -> np.ndarray:
        return self.explicit()


def make_dense(seed: int, d: int, m: int, rho: float = 0.0, exact: bool = True) -> DenseSketch:
    """S[j, c] = N(j d + c) on stream 0; then fp32 and bf16 roundings.

    ``exact`` evaluates log/cos through the C library one value at a time
    (bit-identical to a C implementation); ``exact=False`` uses numpy's
    vectorised log/cos, which is what the Monte-Carlo tests use for speed."""
    if exact:
        S64 = rng.gaussian_exact(seed, rng.STREAM_DENSE, m * d).reshape(m, d)
    else:
        S64 = rng.gaussian_fast(seed, rng.STREAM_DENSE, np.arange(m * d)).reshape(m, d)
    S32 = round_to_f32(S64)
    S16 = round_f32_to_bf16(S32)
    dmag = rng.dither_magnitudes(seed, m, exact) if rho > 0 else None
    return DenseSketch(seed, d, m, rho, S64, S32, S16, dmag=dmag)


def fisher_yates(seed: int, block: int, d: int) -> np.ndarray:
    """P_b: start at the identity; for i = d-1 .. 1 swap P[i] with P[t],
    t = floor(U(b d + i) * (i + 1)) on stream 2 (Fisher and Yates, as in
    Durstenfeld's in-place form)."""
    P = np.arange(d, dtype=np.int64)
    idx = np.arange(block * d, block * d + d, dtype=np.uint64)
    U = rng.uniform53(rng.draw(seed, rng.STREAM_P, idx))
    for i in range(d - 1, 0, -1):
        t = int(np.floor(U[i] * float(i + 1)))
        P[i], P[t] = P[t], P[i]
    return P


def make_fqjl(seed: int, d: int, m: int, rho: float = 0.0, permute: bool = True,
              variant: str = "fqjl", exact: bool = True) -> FqjlSketch:
    """Per block b < m/d: D_b from the top bit of r(seed, 1, b d + c)
    (0 -> +1, 1 -> -1); P_b by Fisher-Yates on stream 2 (the identity when
    ``permute`` is false: the D-FQJL construction has no permutation);
    G_b[c] = fp32(N(b d + c)) on stream 3; with dither (rho > 0) the m
    magnitudes of rng.dither_magnitudes."""
    assert m % d == 0
    nb = m // d
    D = np.empty((nb, d))
    P = np.empty((nb, d), dtype=np.int64)
    G = np.empty((nb, d))
    for b in range(nb):
        r = rng.draw(seed, rng.STREAM_D, np.arange(b * d, b * d + d, dtype=np.uint64))
        D[b] = np.where((r >> np.uint64(63)) == 0, 1.0, -1.0)
        P[b] = fisher_yates(seed, b, d) if permute else np.arange(d)
        G[b] = round_to_f32(rng.gaussian_exact(seed, rng.STREAM_G, d, offset=b * d))
    dmag = rng.dither_magnitudes(seed, m, exact) if rho > 0 else None
    return FqjlSketch(seed, d, m, rho, D, P, G, variant, dmag=dmag)


def make_sketch(seed: int, d: int, m: int, variant: str, rho: float = 0.0, exact: bool = True):
    """variant: "dense"; "fqjl" (permutation, optional dither); "dfqjl" (the
    FQJL page's D-FQJL: no permutation, dither rho > 0); "pfqjl" (its P-FQJL:
    permutation, rho = 0)."""
    if variant == "dense":
        return make_dense(seed, d, m, rho, exact)
    if variant == "fqjl":
        return make_fqjl(seed, d, m, rho, exact=exact)
    if variant == "dfqjl":
        if not rho > 0:
            raise ValueError("D-FQJL is the dithered construction: rho > 0")
        return make_fqjl(seed, d, m, rho, permute=False, variant="dfqjl", exact=exact)
    if variant == "pfqjl":
        if rho != 0:
            raise ValueError("P-FQJL is the undithered construction: rho = 0")
        return make_fqjl(seed, d, m, 0.0, variant="pfqjl")
    raise ValueError(variant)


def fqjl_apply(sk: FqjlSketch, X: np.ndarray) -> np.ndarray:
    """Y = X S^T through the chain, block by block, in the pages' order:
    Rademacher diagonal, Hadamard (scaled 1/sqrt d), permutation, Gaussian
    diagonal, Hadamard."""
    X = np.asarray(X, dtype=np.float64)
    d = sk.d
    out = np.empty((X.shape[0], sk.m))
    for b in range(sk.m // d):
        u = X * sk.D[b][None, :]
        u = fwht(u) / np.sqrt(d)
        u = u[:, sk.P[b]]
        u = u * sk.G[b][None, :]
        out[:, b * d:(b + 1) * d] = fwht(u)
    return out
