"""Distortion of the estimator against m, for the dense sketch and the FQJL
page's two constructions alone (D-FQJL: no permutation, dither 0.1; P-FQJL:
permutation, no dither), measured on the GPU and by the oracle on the same
keys and queries.

The statistic is the RMS of (estimate - q.k) / (||q|| ||k||) over every
(query, key) pair of a scaled 7B-decode cache (4 heads x 2048 keys with
outlier channels, 8 queries per head).  The GPU's curve must equal the
oracle's: every pair's estimate is asserted within the score tolerance
of the oracle's (bits checked against the oracle first), and the RMS values
within 1e-3 of each other;
fall as m grows with a log-log slope in [-0.7, -0.3] (the pages' "error
shrinks like m^-1/2"), and, for the dense sketch, match the closed form
sqrt(((pi/2) - cos^2) / m) averaged over the pairs within 10%.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import bit_quantized_jl_amd as qj
import workloads as wl
from gpu_helpers import bits_np, check_bits, check_scores, inband_slack, to_np_f64
from oracle import qjl as oq
from oracle import sketch as osk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MS = [128, 256, 512, 1024]
VARIANTS = [("dense", 0.0), ("dfqjl", 0.1), ("pfqjl", 0.0)]


def note(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def rms_normalised(est, exact, qn, kn):
    e = (est - exact) / (qn[:, :, None] * kn[:, None, :])
    return float(np.sqrt(np.mean(e * e)))


@pytest.mark.parametrize("variant,rho", VARIANTS, ids=[v for v, _ in VARIANTS])
def test_distortion_curve_gpu_equals_oracle(variant, rho):
    w = wl.DECODE_7B.scaled(batch=1, heads=4, n_k=2048, n_q=8)
    K = wl.make_keys(w, "cpu")
    q = wl.make_queries(w, "cpu")
    Kd, qd = to_np_f64(K), to_np_f64(q)
    G, nq, nk = w.groups, w.n_q, w.n_k
    Kg, qg = Kd.reshape(G, nk, w.d), qd.reshape(G, nq, w.d)
    exact = np.einsum("gid,gtd->git", qg, Kg)
    qn = np.linalg.norm(qg, axis=2)
    kn = np.linalg.norm(Kg, axis=2)
    gpu_curve, ora_curve = [], []
    for m in MS:
        note("distortion", variant, rho, m)
        sk = qj.make_sketch(0, w.d, m, variant, rho)
        norms, bits = qj.quantize_keys(sk, K.to(DEV))
        Sq = qj.project_query(sk, q.to(DEV))
        est = qj.score(sk, Sq, bits, norms, G, nq, nk)
        torch.cuda.synchronize()
        est = to_np_f64(est)
        gpu_curve.append(rms_normalised(est, exact, qn, kn))
        sk.close()
        ref = osk.make_sketch(0, w.d, m, variant, rho)
        rb, rn, mg, _ = oq.quantize(ref, Kd, w.dtype)
        gb = bits_np(bits)
        check_bits(gb, rb, mg, m)
        Sq_ref = oq.project(ref, qd, w.dtype)
        s_ref = oq.score(Sq_ref, rb, rn, m, rho, G, nq, nk)
        # pair by pair: the GPU's estimate against the oracle's
        check_scores(est, s_ref, inband_slack(gb, rb, Sq_ref, rn, m, rho, G, nq, nk))
        ora_curve.append(rms_normalised(s_ref, exact, qn, kn))
    note(variant, "m", MS, "rms gpu", [round(x, 5) for x in gpu_curve],
         "rms oracle", [round(x, 5) for x in ora_curve])
    for a, b in zip(gpu_curve, ora_curve):
        assert abs(a - b) <= 1e-3 * b, (a, b)
    assert all(a > b for a, b in zip(ora_curve, ora_curve[1:]))
    slope = np.polyfit(np.log(MS), np.log(ora_curve), 1)[0]
    note(variant, "log-log slope", round(float(slope), 3))
    assert -0.7 <= slope <= -0.3, slope
    if variant == "dense":
        cos2 = (exact / (qn[:, :, None] * kn[:, None, :])) ** 2
        for m, r in zip(MS, ora_curve):
            closed = math.sqrt(float(np.mean((math.pi / 2) - cos2)) / m)
            assert abs(r / closed - 1) < 0.10, (m, r, closed)
