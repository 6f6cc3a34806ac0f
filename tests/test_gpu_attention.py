"""GPU parity of the decode-step attention on the QJL scores (through the C
ABI) against the float64 oracle (oracle/attention.py).

The fused path (bf16 values, d_v = 128, m one of 128, 256, 512, 1024,
16-byte aligned bits and values) and the plain path (everything else) are
both covered, with ragged key counts, odd query counts, a single key, and
the limits where the softmax weights are uniform.  The tolerance is derived
in gpu_helpers.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import bit_quantized_jl_amd as qj
import workloads as wl
from gpu_helpers import (bits_np, check_attention, check_bits, check_projection, inband_slack,
                         logit_error_bound, to_np_f64)
from oracle import attention as oa
from oracle import qjl as oq
from oracle import sketch as osk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def random_inputs(m, G, nq, nk, dv, vdt, seed, norm_scale=30.0):
    rs = np.random.default_rng(seed)
    bits = wl.make_random_bits(G * nk, m, seed=seed + 100)
    norms = torch.from_numpy(np.abs(rs.standard_normal(G * nk)).astype(np.float32) * norm_scale)
    Sq = torch.from_numpy((rs.standard_normal((G * nq, m)) * 11).astype(np.float32))
    w = wl.Workload("attn", 128, m, "dense", 1, G, nk, nq, "bf16")
    V = wl.make_values(w, "cpu", d_v=dv, dtype=vdt)
    return Sq, bits, norms, V


def run_attention(sk, Sq, bits, norms, V, G, nq, nk, scale, v_offset=0):
    """Run on the GPU; v_offset > 0 passes V at an element offset (unaligned)."""
    Sqd, bd, nd = Sq.to(DEV), bits.to(DEV), norms.to(DEV)
    if v_offset:
        buf = torch.zeros(V.numel() + v_offset, dtype=V.dtype, device=DEV)
        buf[v_offset:].copy_(V.reshape(-1))
        Vd = buf[v_offset:].view(V.shape)
    else:
        Vd = V.to(DEV)
    out = qj.decode_attention(sk, Sqd, bd, nd, Vd, G, nq, nk, scale)
    torch.cuda.synchronize()
    return to_np_f64(out)


def oracle_attention(Sq, bits, norms, V, m, rho, scale, G, nq, nk, slack=None):
    Sqn, bn, nn = to_np_f64(Sq), bits_np(bits), to_np_f64(norms)
    ref = oa.decode_attention(Sqn, bn, nn, to_np_f64(V), m, rho, scale, G, nq, nk)
    s = oq.score(Sqn, bn, nn, m, rho, G, nq, nk)
    dx = logit_error_bound(s, Sqn, nn, m, rho, scale, G, nq, nk, slack)
    return ref, dx


# (m, G, nq, nk, d_v, value dtype): FUSED takes the fused path, PLAIN the
# plain one (float values, d_v != 128, m not in 128, 256, 512, 1024)
FUSED = [(128, 1, 1, 1, 128, "bf16"), (128, 2, 1, 17, 128, "bf16"),
         (256, 3, 1, 1000, 128, "bf16"), (512, 1, 3, 4096, 128, "bf16"),
         (1024, 2, 2, 2049, 128, "bf16"), (256, 1, 1, 50001, 128, "bf16"),
         (256, 5, 4, 257, 128, "bf16"),
         # three or more queries per group: the matrix-core weighted sums
         (128, 2, 8, 1000, 128, "bf16"), (256, 3, 7, 513, 128, "bf16"),
         (512, 2, 6, 2049, 128, "bf16"), (256, 1, 16, 4096, 128, "bf16"),
         (128, 1, 3, 31, 128, "bf16"), (512, 4, 5, 20000, 128, "bf16"),
         (1024, 1, 4, 300, 128, "bf16"),
         # a group per compute unit or more: one workgroup per group writes
         # the result itself (no combine pass), for one, two and four queries
         (256, 256, 1, 777, 128, "bf16"), (256, 300, 2, 129, 128, "bf16"),
         (256, 256, 4, 333, 128, "bf16"), (128, 260, 3, 65, 128, "bf16")]
PLAIN = [(384, 1, 2, 300, 128, "bf16"), (256, 2, 1, 300, 128, "f32"),
         (256, 2, 2, 300, 64, "bf16"), (96, 1, 2, 130, 128, "bf16"),
         (2048, 1, 1, 64, 128, "bf16"), (32, 3, 3, 33, 7, "f32")]


@pytest.mark.parametrize("m,G,nq,nk,dv,vdt", FUSED + PLAIN)
def test_attention_random_bits(m, G, nq, nk, dv, vdt):
    note("attention", m, G, nq, nk, dv, vdt)
    Sq, bits, norms, V = random_inputs(m, G, nq, nk, dv, vdt, seed=m + G + nq + nk)
    scale = 1.0 / math.sqrt(128.0)
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    got = run_attention(sk, Sq, bits, norms, V, G, nq, nk, scale)
    ref, dx = oracle_attention(Sq, bits, norms, V, m, 0.0, scale, G, nq, nk)
    check_attention(got, ref, to_np_f64(V), dx)
    sk.close()


def test_attention_unaligned_values_take_plain_path():
    m, G, nq, nk = 256, 2, 1, 300
    note("attention unaligned V")
    Sq, bits, norms, V = random_inputs(m, G, nq, nk, 128, "bf16", seed=3)
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    scale = 0.1
    got = run_attention(sk, Sq, bits, norms, V, G, nq, nk, scale, v_offset=1)
    ref, dx = oracle_attention(Sq, bits, norms, V, m, 0.0, scale, G, nq, nk)
    check_attention(got, ref, to_np_f64(V), dx)
    sk.close()


@pytest.mark.parametrize("m,nk,dv", [(256, 8191, 128), (512, 1000, 128), (256, 500, 64)])
def test_attention_uniform_weights_give_the_mean(m, nk, dv):
    # scale 0 (or all norms 0) makes every weight 1 / nk: the output is the
    # mean of the value rows, whatever the bits; a dropped or repeated key
    # moves it by about |V_t - mean| / nk, far above this bound
    note("attention uniform", m, nk, dv)
    G, nq = 2, 3
    Sq, bits, norms, V = random_inputs(m, G, nq, nk, dv, "bf16", seed=11)
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    mean = to_np_f64(V).reshape(G, nk, dv).mean(axis=1)
    for zero_norms in (False, True):
        nr = torch.zeros_like(norms) if zero_norms else norms
        sc = 0.3 if zero_norms else 0.0
        got = run_attention(sk, Sq, bits, nr, V, G, nq, nk, sc)
        vmax = np.abs(to_np_f64(V)).max()
        err = np.abs(got - mean[:, None, :]).max()
        assert err <= 2e-6 * vmax, (zero_norms, err)
    sk.close()


def test_attention_dominant_key():
    # one key's logit exceeds every other by more than 100: its value row
    m, G, nq, nk = 256, 1, 1, 777
    note("attention dominant key")
    rs = np.random.default_rng(5)
    Sq = torch.from_numpy(rs.standard_normal((1, m)).astype(np.float32))
    signs = (Sq.numpy()[0] >= 0).astype(np.uint8)
    bits_np_rows = np.zeros((nk, m), dtype=np.uint8)
    bits_np_rows[:] = rs.integers(0, 2, size=(nk, m))
    t_star = 413
    bits_np_rows[t_star] = signs  # aligned with the query: the largest score
    bits = torch.from_numpy(oq.pack_bits(bits_np_rows).view(np.int32))
    norms = torch.full((nk,), 1.0, dtype=torch.float32)
    norms[t_star] = 150.0
    V = wl.make_values(wl.Workload("a", 128, m, "dense", 1, 1, nk, 1, "bf16"), "cpu")
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    got = run_attention(sk, Sq, bits, norms, V, G, nq, nk, 1.0)
    ref, dx = oracle_attention(Sq, bits, norms, V, m, 0.0, 1.0, G, nq, nk)
    s = oq.score(to_np_f64(Sq), bits_np(bits), to_np_f64(norms), m, 0.0, 1, 1, nk)[0, 0]
    assert s[t_star] - np.delete(s, t_star).max() > 100
    check_attention(got, ref, to_np_f64(V), dx)
    assert np.allclose(got[0, 0], to_np_f64(V)[t_star], rtol=0, atol=1e-6)
    sk.close()


def test_attention_errors():
    note("attention errors")
    sk = qj.make_sketch(0, 128, 256, "dense", 0.0)
    Sq = torch.zeros(1, 256, device=DEV)
    bits = torch.zeros(4, 8, dtype=torch.int32, device=DEV)
    norms = torch.zeros(4, device=DEV)
    V = torch.zeros(4, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(qj.QJLError):  # softmax over no keys
        qj.decode_attention(sk, Sq, bits, norms, V, 1, 1, 0, 1.0)
    with pytest.raises(qj.QJLError):
        qj.decode_attention(sk, Sq, bits, norms, V, 1, 1, 4, float("nan"))
    ws = torch.empty(8, dtype=torch.uint8, device=DEV)
    with pytest.raises(qj.QJLError):  # workspace too small
        qj.decode_attention(sk, Sq, bits, norms, V, 1, 1, 4, 1.0, workspace=ws)
    # no queries: nothing to do
    out = torch.full((1, 0, 128), 7.0, device=DEV)
    qj.decode_attention(sk, Sq, bits, norms, V, 1, 0, 4, 1.0, out=out)
    assert qj.decode_attention_workspace_size(sk, 1, 0, 4, 128) == 0
    sk.close()


@pytest.mark.parametrize("w", [wl.DECODE_7B.scaled(batch=1, heads=4, n_k=1000),
                               wl.FQJL_7B_DITHER.scaled(batch=1, heads=2, n_k=700)],
                         ids=lambda w: w.name)
def test_attention_end_to_end(w):
    # quantize -> project -> attention on the GPU; the oracle runs the same
    # pipeline from the same keys, queries and values
    note("attention e2e", w.name)
    K = wl.make_keys(w, "cpu")
    q = wl.make_queries(w, "cpu")
    V = wl.make_values(w, "cpu")
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms, bits = qj.quantize_keys(sk, K.to(DEV))
    Sq = qj.project_query(sk, q.to(DEV))
    scale = 1.0 / math.sqrt(w.d)
    out = qj.decode_attention(sk, Sq, bits, norms, V.to(DEV), w.groups, w.n_q, w.n_k, scale)
    torch.cuda.synchronize()
    ref_sk = osk.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    rb, rn, mg, _ = oq.quantize(ref_sk, to_np_f64(K), w.dtype)
    check_bits(bits_np(bits), rb, mg, w.m)
    Sq_ref = oq.project(ref_sk, to_np_f64(q), w.dtype)
    ref = oa.decode_attention(Sq_ref, rb, rn, to_np_f64(V), w.m, w.rho, scale, w.groups, w.n_q,
                              w.n_k)
    slack = inband_slack(bits_np(bits), rb, Sq_ref, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    s = oq.score(Sq_ref, rb, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    dx = logit_error_bound(s, Sq_ref, rn, w.m, w.rho, scale, w.groups, w.n_q, w.n_k, slack)
    # the GPU's projected query (checked against the oracle's within its own
    # tolerance) differs from the oracle's by dSq, which moves each score by
    # at most c ||k|| sum_j |dSq_j|
    Sq_gpu = to_np_f64(Sq)
    check_projection(Sq_gpu, Sq_ref, to_np_f64(q), w.m)
    dsq = np.abs(Sq_gpu - Sq_ref).sum(axis=1).reshape(w.groups, w.n_q)
    c = oq.estimator_constant(w.m, w.rho)
    kmax = rn.reshape(w.groups, w.n_k).max(axis=1)
    dx = dx + scale * c * kmax[:, None] * dsq
    check_attention(to_np_f64(out), ref, to_np_f64(V), dx)
    sk.close()


def test_full_size_decode_7b_attention():
    # the full decode workload (256 groups x 8192 keys, one query each) in the
    # launch configuration the benchmark times; the oracle recomputes sampled
    # groups from the same random bits, norms, queries and values
    w = wl.DECODE_7B
    note("full attention", w.name)
    m, G, nq, nk = w.m, w.groups, w.n_q, w.n_k
    bits = wl.make_random_bits(G * nk, m, seed=21, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(22)
    norms = torch.randn(G * nk, generator=gen, device=DEV).abs_().mul_(30.0)
    Sq = torch.randn(G * nq, m, generator=gen, device=DEV).mul_(11.0)
    V = wl.make_values(w, DEV)
    sk = qj.make_sketch(w.seed, w.d, m, w.variant, w.rho)
    scale = 1.0 / math.sqrt(w.d)
    out = qj.decode_attention(sk, Sq, bits, norms, V, G, nq, nk, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    rs = np.random.default_rng(3)
    for g in sorted(set([0, G - 1] + rs.choice(G, 4, replace=False).tolist())):
        sl = slice(g * nk, (g + 1) * nk)
        qs = slice(g * nq, (g + 1) * nq)
        ref, dx = oracle_attention(Sq[qs].cpu(), bits[sl].cpu(), norms[sl].cpu(), V[sl].cpu(),
                                   m, w.rho, scale, 1, nq, nk)
        check_attention(to_np_f64(out[g:g + 1]), ref, to_np_f64(V[sl]), dx)
    sk.close()
