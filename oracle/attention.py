"""Decode-step attention on the QJL-estimated scores, in float64.

Test infrastructure only: nothing in the product path imports this module.

Source: the QJL abstract (Zandieh, Daliri, Han) on Majid Daliri's
scholarfeed page, and the KIVI abstract on the same site: the sketched keys
serve the attention of a decoding step, where every cached key is scored
against the new query, the scores are turned into softmax weights, and the
output is the weighted sum of the cached value rows.  Plainest reading of what
the pages leave open:
  * the scores are the QJL estimates of q.k (the `score` of qjl.py), scaled
    by a caller-given factor before the softmax (1/sqrt(d) in the usual
    attention);
  * the softmax runs over all n_k keys of a group, per query; the maximum is
    subtracted first, which changes nothing mathematically;
  * the value rows are not sketched: they are the cached values as given.
"""
from __future__ import annotations

import numpy as np

from .qjl import score


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Softmax along the last axis, float64, maximum subtracted first."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def decode_attention(Sq: np.ndarray, bits: np.ndarray, norms: np.ndarray, V: np.ndarray,
                     m: int, rho: float, scale: float, n_groups: int, n_q: int,
                     n_k: int) -> np.ndarray:
    """out[g, i, :] = sum_t softmax_t(scale * s[g, i, t]) V[g, t, :], with s the
    QJL score of query i of group g against key t.  V: [n_groups * n_k, d_v]."""
    s = score(Sq, bits, norms, m, rho, n_groups, n_q, n_k)
    a = softmax_rows(scale * s)
    V64 = np.asarray(V, dtype=np.float64).reshape(n_groups, n_k, -1)
    return np.einsum("gik,gkd->gid", a, V64)
