"""Shared helpers for the GPU parity tests (tolerances and comparisons).

Tolerances:
  * sign bits: identical, except coordinates whose oracle margin
    |y| / (||k|| sqrt d) is below 1e-5 -- there float32 accumulation may
    legitimately flip a sign; such coordinates are counted and reported;
  * norms: relative 1e-5;
  * projected queries: absolute 1e-5 * ||q|| * sqrt(m);
  * scores (the oracle scoring the GPU's bits in float64):
    |gpu - ref| <= 1e-3 |ref| + 1e-4.
"""
from __future__ import annotations

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


def check_scores(gpu: np.ndarray, ref: np.ndarray) -> None:
    err = np.abs(gpu - ref)
    tol = SCORE_RTOL * np.abs(ref) + SCORE_ATOL
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"score mismatch at {i}: gpu {gpu[i]} ref {ref[i]} "
                             f"({int((err > tol).sum())} of {err.size})")


def check_projection(gpu: np.ndarray, ref: np.ndarray, q: np.ndarray, m: int) -> None:
    qn = np.sqrt((q * q).sum(axis=1))[:, None]
    err = np.abs(gpu - ref)
    assert np.all(err <= 1e-5 * qn * np.sqrt(m) + 1e-30), float(np.max(err / (qn * np.sqrt(m))))
