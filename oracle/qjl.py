"""QJL quantizer and asymmetric inner-product estimator in float64.

Test infrastructure only: nothing in the product path imports this module.

Source: the QJL abstract (Zandieh, Daliri, Han) on Majid Daliri's
scholarfeed page.  A key is JL-projected and only the sign of each sketched
coordinate is kept (1 bit each, no zero-point or scale); the query is
projected by the same matrix and left in full precision; the product of the
two is an unbiased estimate of the inner product.

Plainest reading of what the abstract leaves open (each is one line here):
  * the per-key norm ||k|| is stored beside the bits (one float per key, not
    a per-block zero-point/scale);
  * the estimator is  sqrt(pi/2)/m * ||k|| * <S q, sign(S k)>.  For a
    Gaussian row s, E[sign(s.k) (s.q)] = sqrt(2/pi) q.k/||k||, so this is the
    unique constant that makes it unbiased;
  * sign(0) is taken as +1 (bit 1 <=> y >= 0);
  * bits are packed LSB-first: bit t of 32-bit word w is coordinate 32 w + t.

Dither (the D-FQJL construction on the "Fast Quantized Johnson-Lindenstrauss
Transforms" page, "Key concepts" and "The paper's improvements"): Gaussian
noise of standard deviation rho*||k|| is added to each sketched coordinate
before the sign.  Then E[sign(x + xi) y] = sqrt(2/pi) q.k / (||k||
sqrt(1 + rho^2)), so the estimator gains the factor sqrt(1 + rho^2).
"""
from __future__ import annotations

import math

import numpy as np

from . import rng
from .sketch import DenseSketch, FqjlSketch, fqjl_apply

CHUNK = 1 << 16


def pack_bits(B: np.ndarray) -> np.ndarray:
    """Boolean [n, m] -> uint32 [n, m/32], bit t of word w = column 32 w + t."""
    B = np.asarray(B, dtype=bool)
    n, m = B.shape
    assert m % 32 == 0
    w = B.reshape(n, m // 32, 32).astype(np.uint64)
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    return (w * weights).sum(axis=-1).astype(np.uint32)


def unpack_bits(W: np.ndarray, m: int) -> np.ndarray:
    """uint32 [n, m/32] -> boolean [n, m] (inverse of pack_bits)."""
    W = np.asarray(W).astype(np.uint32).astype(np.uint64)
    shifts = np.arange(32, dtype=np.uint64)
    B = (W[:, :, None] >> shifts) & np.uint64(1)
    return B.reshape(W.shape[0], m).astype(bool)


def project(sk, X: np.ndarray, in_dtype: str) -> np.ndarray:
    """Y = X S^T in float64 (keys or queries, rows of X)."""
    X = np.asarray(X, dtype=np.float64)
    if isinstance(sk, FqjlSketch):
        return fqjl_apply(sk, X)
    S = sk.effective(in_dtype)
    return X @ S.T


def quantize(sk, K: np.ndarray, in_dtype: str, key_index_base: int = 0, key_index=None):
    """Quantize keys.  Returns (bits uint32 [n, m/32], norms float64 [n],
    margin float64 [n, m], Y float64 [n, m]).

    Row i's dither counter is key_index_base + i, or key_index[i] when an
    explicit array of global key indices is given (for sampled rows).

    Y = S k (+ rho ||k|| xi), bit = [Y >= 0], norm = ||k||_2 and
    margin = |Y| / (||k|| sqrt(d)): how far a coordinate is from the sign
    flip, relative to the scale of a coordinate.  A key of norm 0 has Y = 0
    exactly and margin +inf.
    """
    K = np.asarray(K, dtype=np.float64)
    n, d = K.shape
    m = sk.m
    bits = np.empty((n, m // 32), dtype=np.uint32)
    norms = np.sqrt((K * K).sum(axis=1))
    margin = np.empty((n, m))
    Yall = np.empty((n, m))
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        Y = project(sk, K[s:e], in_dtype)
        if sk.rho > 0:
            ids = (np.arange(key_index_base + s, key_index_base + e) if key_index is None
                   else np.asarray(key_index)[s:e])
            xi = rng.dither(sk.seed, ids, m, sk.dmag)
            Y = Y + sk.rho * norms[s:e, None] * xi
        bits[s:e] = pack_bits(Y >= 0)
        scale = norms[s:e, None] * math.sqrt(d)
        with np.errstate(divide="ignore", invalid="ignore"):
            mg = np.abs(Y) / scale
        mg[np.broadcast_to(scale == 0, mg.shape)] = np.inf
        margin[s:e] = mg
        Yall[s:e] = Y
    return bits, norms, margin, Yall


def estimator_constant(m: int, rho: float) -> float:
    """sqrt(pi/2) * sqrt(1 + rho^2) / m."""
    return math.sqrt(math.pi / 2.0) * math.sqrt(1.0 + rho * rho) / m


def score(Sq: np.ndarray, bits: np.ndarray, norms: np.ndarray, m: int, rho: float,
          n_groups: int, n_q: int, n_k: int) -> np.ndarray:
    """scores[g, i, t] = c * norm[g, t] * sum_j (2 bit[g, t, j] - 1) Sq[g, i, j]."""
    Sq = np.asarray(Sq, dtype=np.float64).reshape(n_groups, n_q, m)
    norms = np.asarray(norms, dtype=np.float64).reshape(n_groups, n_k)
    bits = np.asarray(bits).reshape(n_groups * n_k, m // 32)
    c = estimator_constant(m, rho)
    out = np.empty((n_groups, n_q, n_k))
    for g in range(n_groups):
        sg = 2.0 * unpack_bits(bits[g * n_k:(g + 1) * n_k], m).astype(np.float64) - 1.0
        out[g] = c * (Sq[g] @ sg.T) * norms[g][None, :]
    return out


def score_keys(Sq_row: np.ndarray, bits_rows: np.ndarray, norms_rows: np.ndarray,
               m: int, rho: float) -> np.ndarray:
    """Scores of one query against a few keys (used for sampled checks)."""
    sg = 2.0 * unpack_bits(np.asarray(bits_rows).reshape(-1, m // 32), m).astype(np.float64) - 1.0
    return estimator_constant(m, rho) * np.asarray(norms_rows, np.float64) * (sg @ np.asarray(Sq_row, np.float64))


def estimate_inner_product(sk, q: np.ndarray, k: np.ndarray, in_dtype: str = "f32",
                           key_index: int = 0) -> float:
    """The whole pipeline for one (q, k) pair: quantize k, project q, score."""
    bits, norms, _, _ = quantize(sk, k[None, :], in_dtype, key_index)
    Sq = project(sk, q[None, :], in_dtype)
    return float(score(Sq, bits, norms, sk.m, sk.rho, 1, 1, 1)[0, 0, 0])
