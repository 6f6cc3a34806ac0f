"""Shared helpers for the GPU parity tests (tolerances and comparisons).

Tolerances:
  * sign bits: identical, except coordinates whose oracle margin
    |y| / (||k|| sqrt d) is below 1e-5 -- there float32 accumulation may
    legitimately flip a sign; such coordinates are counted and reported;
  * norms: relative 1e-5;
  * projected queries: absolute 1e-5 * ||q|| * sqrt(m);
  * scores: |gpu - ref| <= 1e-3 |ref| + 1e-4, where ref is the oracle's
    float64 score of the oracle's own bits, norms and projected query; a sign
    bit that legitimately differs inside the band adds its whole effect on
    the estimate, 2 c ||k|| |Sq_j| (c the estimator constant), to the bound;
  * decode attention: a change dx_t in logit t moves a softmax-weighted mean
    of the value rows by at most 2 max_t |dx_t| max|V| (first order), so
    |gpu - ref| <= 2 dx max|V| + 1e-5 max|V| + 1e-5 |ref| per group, dx
    bounding the float32 error of the logits: scale (8 eps |s| +
    eps c ||k|| m max|Sq|) with eps = 2^-24 (the products that form a logit,
    and the query's fixed-point digits), plus the in-band slack above; the
    1e-5 terms cover the float32 weighted sums.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

from oracle import qjl as oq

BAND = 1e-5
NORM_RTOL = 1e-5
SCORE_RTOL = 1e-3
SCORE_ATOL = 1e-4


def to_np_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint32)


def check_bits(gpu_bits: np.ndarray, ref_bits: np.ndarray, margin: np.ndarray, m: int,
               band: float = BAND) -> int:
    """Assert bits agree outside the band; return the in-band mismatch count."""
    g = oq.unpack_bits(gpu_bits, m)
    r = oq.unpack_bits(ref_bits, m)
    diff = g != r
    bad = diff & (margin >= band)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} sign bits differ outside the 1e-5 band, "
                             f"first at {idx.tolist()} margins {margin[bad][:5].tolist()}")
    return int(diff.sum())


def check_norms(gpu: np.ndarray, ref: np.ndarray) -> None:
    err = np.abs(gpu - ref)
    tol = NORM_RTOL * np.abs(ref)
    assert np.all(err <= tol), f"norm error {np.max(err / np.maximum(ref, 1e-30))}"


def inband_slack(gpu_bits: np.ndarray, ref_bits: np.ndarray, Sq: np.ndarray,
                 norms: np.ndarray, m: int, rho: float, G: int, nq: int, nk: int) -> np.ndarray:
    """[G, nq, nk] bound on how much sign bits that differ from the oracle's
    (only ever inside the band, which check_bits asserts) move each score."""
    flip = (oq.unpack_bits(gpu_bits, m) != oq.unpack_bits(ref_bits, m)).astype(np.float64)
    c = oq.estimator_constant(m, rho)
    F = flip.reshape(G, nk, m)
    A = np.abs(np.asarray(Sq, dtype=np.float64)).reshape(G, nq, m)
    nr = np.asarray(norms, dtype=np.float64).reshape(G, 1, nk)
    return 2.0 * c * nr * np.einsum("gij,gtj->git", A, F)


def check_scores(gpu: np.ndarray, ref: np.ndarray, slack=None) -> None:
    err = np.abs(gpu - ref)
    tol = SCORE_RTOL * np.abs(ref) + SCORE_ATOL
    if slack is not None:
        tol = tol + np.reshape(slack, tol.shape)
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"score mismatch at {i}: gpu {gpu[i]} ref {ref[i]} "
                             f"({int((err > tol).sum())} of {err.size})")


def check_projection(gpu: np.ndarray, ref: np.ndarray, q: np.ndarray, m: int) -> None:
    qn = np.sqrt((q * q).sum(axis=1))[:, None]
    err = np.abs(gpu - ref)
    assert np.all(err <= 1e-5 * qn * np.sqrt(m) + 1e-30), float(np.max(err / (qn * np.sqrt(m))))


EPS32 = 2.0 ** -24


def logit_error_bound(scores: np.ndarray, Sq: np.ndarray, norms: np.ndarray, m: int,
                      rho: float, scale: float, G: int, nq: int, nk: int,
                      slack=None) -> np.ndarray:
    """[G, nq] bound on the float32 error of the logits scale * s of a row."""
    s = np.abs(np.asarray(scores, dtype=np.float64)).reshape(G, nq, nk)
    c = oq.estimator_constant(m, rho)
    kmax = np.abs(np.asarray(norms, dtype=np.float64)).reshape(G, nk).max(axis=1)
    qmax = np.abs(np.asarray(Sq, dtype=np.float64)).reshape(G, nq, m).max(axis=2)
    dx = abs(scale) * (8 * EPS32 * s.max(axis=2) + EPS32 * c * kmax[:, None] * m * qmax)
    if slack is not None:
        dx = dx + abs(scale) * np.reshape(slack, (G, nq, nk)).max(axis=2)
    return dx


def check_attention(gpu: np.ndarray, ref: np.ndarray, V: np.ndarray, dx: np.ndarray) -> None:
    """gpu, ref: [G, nq, d_v]; V: [G * nk, d_v]; dx: [G, nq]."""
    G = ref.shape[0]
    vmax = np.abs(np.asarray(V, dtype=np.float64)).reshape(G, -1).max(axis=1)
    tol = ((2 * dx + 1e-5) * vmax[:, None])[:, :, None] + 1e-5 * np.abs(ref)
    err = np.abs(gpu - ref)
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"attention mismatch at {i}: gpu {gpu[i]} ref {ref[i]} tol {tol[i]} "
                             f"({int((err > tol).sum())} of {err.size})")


# ---------------------------------------------------------------- reporting
# (config, coordinates compared, in-band sign differences) of the parity
# checks that ran; the conftest's terminal summary prints one line per entry.
INBAND_REPORT: list = []


def report_inband(name: str, coords: int, inband: int) -> None:
    INBAND_REPORT.append((name, int(coords), int(inband)))


# ------------------------------------------------------------ whole outputs
def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _one_blas_thread():
    """A context in which numpy's BLAS runs single-threaded (the chunks are
    already spread over a thread pool)."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:  # threadpoolctl missing: run as is
        import contextlib
        return contextlib.nullcontext()


def oracle_check_all_rows(ref, K: torch.Tensor, dtype: str, gpu_bits: np.ndarray,
                          gpu_norms: np.ndarray, key_index_base: int = 0, chunk: int = 8192):
    """Every row of a quantized cache against the oracle.

    The oracle quantizes K (a host tensor, [n, d]) chunk by chunk on a
    thread pool; each chunk's bits and norms are compared with the GPU's
    (check_bits / check_norms).  Returns (in-band sign differences, oracle
    bits [n, m/32], oracle norms [n])."""
    n = K.shape[0]
    m = ref.m
    rb_all = np.empty((n, m // 32), dtype=np.uint32)
    rn_all = np.empty(n, dtype=np.float64)

    def work(s):
        e = min(n, s + chunk)
        Kd = K[s:e].to(torch.float64).numpy()
        rb, rn, mg, _ = oq.quantize(ref, Kd, dtype, key_index_base=key_index_base + s)
        nb = check_bits(gpu_bits[s:e], rb, mg, m)
        check_norms(gpu_norms[s:e], rn)
        rb_all[s:e] = rb
        rn_all[s:e] = rn
        return nb

    with _one_blas_thread(), cf.ThreadPoolExecutor(_workers()) as ex:
        inband = sum(ex.map(work, range(0, n, chunk)))
    return inband, rb_all, rn_all


def oracle_check_all_scores(ref, q: torch.Tensor, dtype: str, gpu_Sq: np.ndarray,
                            gpu_scores: np.ndarray, gpu_bits: np.ndarray, rb: np.ndarray,
                            rn: np.ndarray, rho: float, G: int, nq: int, nk: int) -> None:
    """Every group's scores against the oracle's, formed from the oracle's own
    projection of the queries and its own bits and norms (rb, rn: all rows);
    a sign that differs inside the band widens its scores' bound by its whole
    effect (inband_slack).  The projections are checked diagnostically."""
    m = ref.m
    qd_all = q.to(torch.float64).numpy()

    def work(g):
        qd = qd_all[g * nq:(g + 1) * nq]
        Sq_ref = oq.project(ref, qd, dtype)
        check_projection(gpu_Sq[g * nq:(g + 1) * nq], Sq_ref, qd, m)
        sl = slice(g * nk, (g + 1) * nk)
        s_ref = oq.score(Sq_ref, rb[sl], rn[sl], m, rho, 1, nq, nk)
        slack = inband_slack(gpu_bits[sl], rb[sl], Sq_ref, rn[sl], m, rho, 1, nq, nk)
        check_scores(gpu_scores[g], s_ref[0], slack[0])

    with _one_blas_thread(), cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(work, range(G)))
