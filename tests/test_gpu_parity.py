"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Small and medium shapes are checked element by element, and so are the
full-size workloads (run in the same launch configuration the benchmark
times): every row of their caches and every score, against the oracle run
chunk by chunk on a thread pool.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import bit_quantized_jl_amd as qj
import workloads as wl
from gpu_helpers import (bits_np, check_bits, check_norms, check_projection, check_scores,
                         inband_slack, oracle_check_all_rows, oracle_check_all_scores,
                         report_inband, to_np_f64)
from oracle import qjl as oq
from oracle import sketch as osk

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


_osk_cache: dict = {}


def oracle_sketch(seed, d, m, variant, rho):
    key = (seed, d, m, variant, rho)
    if key not in _osk_cache:
        _osk_cache[key] = osk.make_sketch(seed, d, m, variant, rho)
    return _osk_cache[key]


def run_quantize_case(w: wl.Workload, n_k: int | None = None, base: int = 0):
    note("quantize", w.name, w.d, w.m, w.variant, w.dtype, w.rho, n_k)
    K = wl.make_keys(w, "cpu", n_k=n_k).to(DEV)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms, bits = qj.quantize_keys(sk, K, key_index_base=base)
    torch.cuda.synchronize()
    ref = oracle_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Kd = to_np_f64(K)
    rb, rn, mg, _ = oq.quantize(ref, Kd, w.dtype, key_index_base=base)
    nband = check_bits(bits_np(bits), rb, mg, w.m)
    check_norms(to_np_f64(norms), rn)
    sk.close()
    return nband, K, bits, norms, rb, rn


QUANT_CASES = [
    wl.TINY,
    wl.DECODE_7B.scaled(batch=1, heads=4, n_k=1000),
    wl.LONG_CTX.scaled(heads=2, n_k=1531),
    wl.PREFILL.scaled(batch=1, heads=3, n_k=777),
    wl.FQJL_7B.scaled(batch=1, heads=2, n_k=1000),
    wl.FQJL_7B_DITHER.scaled(batch=1, heads=2, n_k=1000),
    wl.DFQJL_7B.scaled(batch=1, heads=2, n_k=1000),
    wl.PFQJL_7B.scaled(batch=1, heads=2, n_k=1000),
]


@pytest.mark.parametrize("w", QUANT_CASES, ids=lambda w: w.name)
def test_quantize_workloads_scaled(w):
    nband, K, *_ = run_quantize_case(w)
    note("in-band sign differences:", nband)
    report_inband(f"{w.name} ({K.shape[0]} keys)", K.shape[0] * w.m, nband)


SHAPES = (
    [("dense", d, m, dt, 0.0) for d in (16, 64, 100, 128, 256) for m in (32, 96, 512)
     for dt in ("f32", "bf16")]
    + [("dense", 128, 256, "bf16", 0.5), ("dense", 64, 128, "f32", 0.1)]
    + [("dense", d, m, "bf16", 0.0) for (d, m) in ((64, 128), (64, 256), (128, 128))]  # MFMA
    + [("fqjl", d, m, dt, rho) for (d, m) in ((8, 32), (16, 32), (16, 64), (32, 32), (32, 96),
                                              (64, 64), (64, 256), (128, 128), (128, 512))
       for dt in ("f32", "bf16") for rho in (0.0, 0.3)]
    + [("dfqjl", d, m, dt, 0.1) for (d, m) in ((8, 32), (16, 64), (32, 96), (64, 256), (128, 128),
                                                (128, 512)) for dt in ("f32", "bf16")]
    + [("pfqjl", d, m, dt, 0.0) for (d, m) in ((16, 32), (64, 192), (128, 256))
       for dt in ("f32", "bf16")]
    # d = 256: four lanes per row (one and two blocks per key)
    + [("fqjl", 256, m, dt, rho) for m in (256, 512) for dt in ("f32", "bf16")
       for rho in (0.0, 0.3)]
    + [("dfqjl", 256, m, dt, 0.1) for m in (256, 512) for dt in ("f32", "bf16")]
    + [("pfqjl", 256, 512, dt, 0.0) for dt in ("f32", "bf16")]
)


@pytest.mark.parametrize("variant,d,m,dt,rho", SHAPES)
def test_quantize_shapes(variant, d, m, dt, rho):
    w = wl.Workload(f"shape_{variant}_{d}_{m}_{dt}_{rho}", d, m, variant, 1, 1, 203, 5, dt,
                    "normal", rho, seed=3)
    run_quantize_case(w, base=11)


@pytest.mark.parametrize("variant,d,m,rho", [
    ("dense", 64, 128, 0.0), ("dense", 64, 256, 0.0), ("dense", 64, 512, 0.0),
    ("dense", 128, 128, 0.0), ("dense", 128, 256, 0.0), ("dense", 128, 512, 0.0),
    ("fqjl", 128, 128, 0.0), ("fqjl", 128, 256, 0.2), ("fqjl", 128, 512, 0.0),
    ("dfqjl", 128, 256, 0.1), ("dfqjl", 128, 512, 0.1), ("fqjl", 256, 512, 0.3)])
def test_quantize_persistent_kernel_shapes(variant, d, m, rho):
    # More than 16384 bf16 keys (a ragged count): the persistent matrix-core
    # quantizers with the operand image staged in LDS, for every shape they
    # serve (shorter calls take the short-call kernels).
    w = wl.Workload(f"persistent_{variant}_{d}_{m}", d, m, variant, 1, 1, 16384 + 1357, 5,
                    "bf16", "normal", rho, seed=4)
    run_quantize_case(w, base=3)


@pytest.mark.parametrize("variant,d,m,dt,n", [
    ("fqjl", 128, 256, "bf16", 20000),   # persistent matrix-core kernel
    ("fqjl", 128, 256, "bf16", 300),     # short-call matrix-core kernel
    ("dfqjl", 128, 512, "bf16", 300),
    ("fqjl", 128, 256, "f32", 300),      # two lanes per row
    ("fqjl", 64, 128, "bf16", 300),      # one lane per row
    ("fqjl", 256, 512, "bf16", 300),     # four lanes per row
    ("fqjl", 16, 64, "f32", 300),        # small d
    ("dense", 128, 256, "bf16", 300)])   # dense sketch with dither
def test_dither_counters_at_large_key_indices(variant, d, m, dt, n):
    # The dither's sign-word counter is (key index) * ceil(m/64) + word in 64
    # bits: key indices past 2^40, whose products pass 2^42, must give the
    # oracle's draws in every kernel that dithers.
    w = wl.Workload(f"bigindex_{variant}_{d}_{m}_{dt}", d, m, variant, 1, 1, n, 5, dt, "normal",
                    0.2, seed=8)
    run_quantize_case(w, base=(1 << 40) + 12345)


@pytest.mark.parametrize("d,m", [(64, 128), (64, 256), (128, 128), (128, 256)])
def test_dense_schedules_identical(monkeypatch, d, m):
    # The dense quantizer's register schedules (QJL_DENSE_SCHEDULE): each one's
    # bits and norms equal the default schedule's, whose every row is checked
    # against the oracle.  The key count gives each wave of the persistent
    # grid several tiles, an odd number for some waves and an even number for
    # others (both exits of the prefetching loop), and a short last tile.
    n = 3 * 2048 * 128 + 777
    w = wl.Workload(f"schedules_{d}_{m}", d, m, "dense", 1, 1, n, 5, "bf16", "normal", 0.0,
                    seed=6)
    note("dense schedules", d, m, n)
    Kh = wl.make_keys(w, "cpu")
    K = Kh.to(DEV)
    sk = qj.make_sketch(w.seed, d, m, "dense", 0.0)
    monkeypatch.delenv("QJL_DENSE_SCHEDULE", raising=False)
    n0, b0 = qj.quantize_keys(sk, K)
    torch.cuda.synchronize()
    ref = oracle_sketch(w.seed, d, m, "dense", 0.0)
    oracle_check_all_rows(ref, Kh, "bf16", bits_np(b0), to_np_f64(n0))
    for schedule in ("prefetch", "rt4", "immediate"):
        monkeypatch.setenv("QJL_DENSE_SCHEDULE", schedule)
        n1, b1 = qj.quantize_keys(sk, K)
        torch.cuda.synchronize()
        assert torch.equal(b1, b0), schedule
        assert torch.equal(n1, n0), schedule
    sk.close()


@pytest.mark.parametrize("variant,d,m,dt,nq", [
    ("dense", 128, 256, "f32", 37), ("dense", 128, 256, "bf16", 37), ("dense", 100, 96, "bf16", 37),
    ("dense", 16, 512, "f32", 37), ("dense", 128, 256, "bf16", 300), ("dense", 64, 128, "bf16", 33),
    ("dense", 256, 64, "bf16", 65), ("dense", 48, 192, "bf16", 31), ("dense", 16, 64, "bf16", 1),
    ("dense", 128, 512, "bf16", 70), ("fqjl", 128, 256, "bf16", 37), ("fqjl", 8, 32, "f32", 37),
    ("fqjl", 64, 192, "f32", 37), ("fqjl", 128, 512, "bf16", 37), ("dfqjl", 128, 256, "bf16", 37),
    ("dfqjl", 16, 64, "f32", 37), ("pfqjl", 128, 256, "bf16", 37), ("fqjl", 128, 128, "bf16", 70),
    ("fqjl", 128, 256, "bf16", 300), ("dfqjl", 128, 512, "bf16", 1),
    ("fqjl", 256, 512, "bf16", 37), ("fqjl", 256, 256, "f32", 37), ("dfqjl", 256, 256, "bf16", 37),
    ("pfqjl", 256, 512, "f32", 37), ("fqjl", 256, 512, "bf16", 300)])
def test_project_query(variant, d, m, dt, nq):
    note("project", variant, d, m, dt, nq)
    rho = 0.1 if variant == "dfqjl" else 0.0  # queries are never dithered
    w = wl.Workload("proj", d, m, variant, 1, 1, 1, nq, dt, seed=5)
    q = wl.make_queries(w, "cpu").to(DEV)
    sk = qj.make_sketch(5, d, m, variant, rho)
    Sq = qj.project_query(sk, q)
    torch.cuda.synchronize()
    ref = oracle_sketch(5, d, m, variant, rho)
    qd = to_np_f64(q)
    check_projection(to_np_f64(Sq), oq.project(ref, qd, dt), qd, m)
    sk.close()


@pytest.mark.parametrize("variant", ["dense", "fqjl", "dfqjl"])
def test_project_query_unaligned_output(variant):
    # Sq_out 4 bytes past a 16-byte boundary takes the vector kernels instead
    # of the matrix-core ones; both agree with the oracle.
    note("project, unaligned Sq", variant)
    d, m, nq = 128, 256, 45
    rho = 0.1 if variant == "dfqjl" else 0.0
    q = torch.randn(nq, d, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    sk = qj.make_sketch(12, d, m, variant, rho)
    flat = torch.empty(nq * m + 4, dtype=torch.float32, device=DEV)
    Sq = flat[1:1 + nq * m].view(nq, m)
    assert Sq.data_ptr() % 16 == 4
    qj.project_query(sk, q.to(DEV), Sq_out=Sq)
    torch.cuda.synchronize()
    qd = to_np_f64(q)
    check_projection(to_np_f64(Sq), oq.project(oracle_sketch(12, d, m, variant, rho), qd, "bf16"),
                     qd, m)
    sk.close()


SENTINEL_BITS = 0x5A5A5A5A
SENTINEL_NORM = -7.0


@pytest.mark.parametrize("variant,d,m,dt,rho,G,kpg,cap,first", [
    ("dense", 128, 256, "bf16", 0.0, 37, 1, 300, 299),    # decode append, matrix cores
    ("dense", 128, 256, "bf16", 0.0, 5, 70, 200, 17),     # prefill into spare capacity
    ("dense", 128, 512, "bf16", 0.0, 3, 129, 129, 0),     # whole groups
    ("dense", 128, 256, "f32", 0.0, 9, 3, 11, 8),         # float32 keys (generic kernel)
    ("dense", 96, 64, "bf16", 0.3, 4, 33, 40, 5),         # dithered dense (generic kernel)
    ("fqjl", 128, 256, "bf16", 0.0, 64, 1, 50, 13),       # matrix-core first stage
    ("fqjl", 128, 256, "bf16", 0.1, 6, 45, 64, 19),       # with dither
    ("dfqjl", 128, 256, "bf16", 0.1, 7, 2, 9, 7),
    ("fqjl", 128, 512, "bf16", 0.1, 11, 3, 40, 20),       # four blocks per key, dither
    ("pfqjl", 128, 512, "bf16", 0.0, 5, 33, 70, 37),
    ("fqjl", 128, 128, "bf16", 0.0, 9, 2, 20, 5),         # one block: the persistent kernel
    ("dense", 128, 256, "bf16", 0.0, 2, 9000, 9100, 50),  # > 16384 keys: persistent kernels
    ("fqjl", 128, 256, "bf16", 0.1, 2, 9000, 9100, 50),
    ("fqjl", 256, 512, "bf16", 0.1, 5, 3, 10, 4),         # four lanes per row
    ("dfqjl", 256, 256, "f32", 0.2, 3, 20, 33, 13),
    ("fqjl", 64, 192, "f32", 0.2, 5, 17, 17, 0),          # one row per lane
    ("fqjl", 16, 64, "f32", 0.0, 3, 5, 12, 2)])           # narrow blocks
def test_quantize_into_cache(variant, d, m, dt, rho, G, kpg, cap, first):
    # Rows g * cap + first + i get key i of group g, quantized as the oracle
    # does with dither key index base + that row; every other row keeps its
    # sentinel.
    _into_cache_case(variant, d, m, dt, rho, G, kpg, cap, first, 1234)


@pytest.mark.parametrize("variant,d,m,dt,rho,G,kpg,cap,first", [
    ("fqjl", 128, 256, "bf16", 0.1, 2, 9000, 9100, 50),   # persistent kernel, row map
    ("fqjl", 128, 256, "bf16", 0.1, 6, 45, 64, 19),       # short-call kernel, row map
    ("dense", 96, 64, "bf16", 0.3, 4, 33, 40, 5)])        # generic kernel
def test_quantize_into_cache_at_large_key_indices(variant, d, m, dt, rho, G, kpg, cap, first):
    # The same with a key index base past 2^40: the mapped rows' 64-bit
    # dither counters.
    _into_cache_case(variant, d, m, dt, rho, G, kpg, cap, first, (1 << 40) + 1234)


def _into_cache_case(variant, d, m, dt, rho, G, kpg, cap, first, base):
    note("quantize into cache", variant, d, m, dt, rho, G, kpg, cap, first, base)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(G * 7 + kpg + cap + first)
    K = (torch.randn(G * kpg, d, generator=gen) * 2).to(tdt)
    sk = qj.make_sketch(4, d, m, variant, rho)
    W = m // 32
    norms = torch.full((G * cap,), SENTINEL_NORM, dtype=torch.float32, device=DEV)
    bits = torch.full((G * cap, W), SENTINEL_BITS, dtype=torch.int32, device=DEV)
    qj.quantize_keys_into(sk, K.to(DEV), G, norms, bits, cap, first, key_index_base=base)
    torch.cuda.synchronize()
    rows = (np.arange(G)[:, None] * cap + first + np.arange(kpg)[None, :]).reshape(-1)
    ref = oracle_sketch(4, d, m, variant, rho)
    rb, rn, mg, _ = oq.quantize(ref, to_np_f64(K), dt, key_index=base + rows)
    got_b, got_n = bits_np(bits), to_np_f64(norms)
    check_bits(got_b[rows], rb, mg, m)
    check_norms(got_n[rows], rn)
    untouched = np.ones(G * cap, dtype=bool)
    untouched[rows] = False
    assert np.all(got_b[untouched] == np.uint32(SENTINEL_BITS))
    assert np.all(got_n[untouched] == SENTINEL_NORM)
    sk.close()


@pytest.mark.parametrize("variant,rho", [("fqjl", 0.0), ("fqjl", 0.2), ("dfqjl", 0.1),
                                         ("dense", 0.0)])
def test_bits_buffer_alignment_paths(variant, rho):
    # bits_out 4 bytes past a 16-byte boundary takes the vector kernels
    # (FQJL: fqjl128_kernel, dense: the generic kernel) instead of the
    # matrix-core ones; both agree with the oracle.
    note("misaligned bits", variant, rho)
    d, m, n = 128, 256, 777
    W = m // 32
    K = (torch.randn(n, d, generator=torch.Generator().manual_seed(3)) * 1.7).to(torch.bfloat16)
    sk = qj.make_sketch(6, d, m, variant, rho)
    flat = torch.empty(n * W + 4, dtype=torch.int32, device=DEV)
    bits = flat[1:1 + n * W].view(n, W)
    assert bits.data_ptr() % 16 == 4
    norms = torch.empty(n, dtype=torch.float32, device=DEV)
    qj.quantize_keys(sk, K.to(DEV), key_index_base=5, norms_out=norms, bits_out=bits)
    torch.cuda.synchronize()
    ref = oracle_sketch(6, d, m, variant, rho)
    rb, rn, mg, _ = oq.quantize(ref, to_np_f64(K), "bf16", key_index_base=5)
    check_bits(bits_np(bits.contiguous()), rb, mg, m)
    check_norms(to_np_f64(norms), rn)
    sk.close()


@pytest.mark.parametrize("variant,dt,rho", [("fqjl", "bf16", 0.0), ("fqjl", "f32", 0.3),
                                            ("dfqjl", "bf16", 0.1)])
def test_fqjl256_unaligned_keys(variant, dt, rho):
    # d = 256 keys one element past a 16-byte boundary: the four-lanes-per-row
    # kernel with element loads instead of 16-byte vectors; same oracle bar.
    note("fqjl d=256 unaligned keys", variant, dt, rho)
    d, m, n = 256, 512, 301
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    K = (torch.randn(n, d, generator=torch.Generator().manual_seed(17)) * 0.7).to(tdt)
    flat = torch.empty(n * d + 1, dtype=tdt, device=DEV)
    Ku = flat[1:].view(n, d)
    Ku.copy_(K.to(DEV))
    assert Ku.data_ptr() % 16 != 0
    sk = qj.make_sketch(13, d, m, variant, rho)
    norms, bits = qj.quantize_keys(sk, Ku, key_index_base=40)
    Sq = qj.project_query(sk, Ku)
    torch.cuda.synchronize()
    ref = oracle_sketch(13, d, m, variant, rho)
    Kd = to_np_f64(K)
    rb, rn, mg, _ = oq.quantize(ref, Kd, dt, key_index_base=40)
    check_bits(bits_np(bits), rb, mg, m)
    check_norms(to_np_f64(norms), rn)
    check_projection(to_np_f64(Sq), oq.project(ref, Kd, dt), Kd, m)
    sk.close()


@pytest.mark.parametrize("variant,rho,m,G,T", [("dense", 0.0, 256, 24, 9), ("fqjl", 0.1, 256, 24, 9),
                                               ("dense", 0.0, 256, 64, 300),
                                               ("dense", 0.0, 512, 40, 420),
                                               ("fqjl", 0.2, 256, 64, 300),
                                               ("fqjl", 0.0, 512, 40, 420),
                                               ("fqjl", 0.0, 128, 48, 380),
                                               # dithered: persistent kernel (whole cache)
                                               # against the short-call kernel (appends)
                                               ("dfqjl", 0.1, 256, 64, 300),
                                               ("fqjl", 0.3, 128, 48, 380),
                                               ("fqjl", 0.1, 512, 40, 420)])
def test_cache_built_by_appends_equals_whole(variant, rho, m, G, T):
    # Appending one key per group per step, then a block of four, fills the
    # cache exactly as one call over the whole cache (dither counters given
    # by the cache row).  The cases with G T > 16384 keys compare the
    # persistent matrix-core kernel (whole cache) with the short-call kernel
    # (appends): the same sums in the same order, so the same bits, the
    # dither included (at m = 128 the appends take the persistent kernel's
    # row-mapped variant).
    note("appends vs whole", variant, rho, m, G, T)
    d = 128
    gen = torch.Generator().manual_seed(5)
    cache_keys = (torch.randn(G, T, d, generator=gen) * 1.5).to(torch.bfloat16).to(DEV)
    sk = qj.make_sketch(2, d, m, variant, rho)
    whole_n, whole_b = qj.quantize_keys(sk, cache_keys.reshape(G * T, d), key_index_base=77)
    norms = torch.full((G * T,), SENTINEL_NORM, dtype=torch.float32, device=DEV)
    bits = torch.full((G * T, m // 32), SENTINEL_BITS, dtype=torch.int32, device=DEV)
    for t in range(T - 4):
        qj.quantize_keys_into(sk, cache_keys[:, t].contiguous(), G, norms, bits, T, t,
                              key_index_base=77)
    qj.quantize_keys_into(sk, cache_keys[:, T - 4:].reshape(G * 4, d).contiguous(), G, norms, bits,
                          T, T - 4, key_index_base=77)
    torch.cuda.synchronize()
    assert torch.equal(bits, whole_b)
    assert torch.equal(norms, whole_n)
    sk.close()


@pytest.mark.parametrize("variant,m,rho", [("dense", 256, 0.0), ("dense", 512, 0.0),
                                           ("fqjl", 256, 0.0), ("fqjl", 512, 0.1),
                                           ("dfqjl", 256, 0.1), ("fqjl", 128, 0.2)])
def test_call_size_does_not_change_bits(variant, m, rho):
    # The first 3000 keys quantized alone (short-call kernels) and as part of
    # a 20000-key call (persistent kernels): identical bits and norms.
    note("call size", variant, m, rho)
    d, n = 128, 20000
    K = (torch.randn(n, d, generator=torch.Generator().manual_seed(m + 3)) * 1.3)
    K = K.to(torch.bfloat16).to(DEV)
    sk = qj.make_sketch(21, d, m, variant, rho)
    n_all, b_all = qj.quantize_keys(sk, K, key_index_base=9)
    n_few, b_few = qj.quantize_keys(sk, K[:3000].contiguous(), key_index_base=9)
    torch.cuda.synchronize()
    assert torch.equal(b_few, b_all[:3000])
    assert torch.equal(n_few, n_all[:3000])
    sk.close()


def test_quantize_into_cache_errors():
    note("quantize into cache errors")
    sk = qj.make_sketch(0, 128, 256, "dense", 0.0)
    lib = qj.load()
    K = torch.randn(4, 128, device=DEV).to(torch.bfloat16)
    nb = torch.empty(64, device=DEV)
    bb = torch.empty((64, 8), dtype=torch.int32, device=DEV)
    call = lambda G, kpg, cap, first, base=0: lib.qjl_quantize_keys_into(
        sk.handle, K.data_ptr(), 1, G, kpg, cap, first, base, nb.data_ptr(), bb.data_ptr(), None)
    assert call(2, 2, 8, 7) == qj.ERR_INVALID_ARGUMENT      # rows past the group's slice
    assert call(2, 2, 8, -1) == qj.ERR_INVALID_ARGUMENT     # negative first row
    assert call(-1, 2, 8, 0) == qj.ERR_INVALID_ARGUMENT
    assert call(2, 2, 8, 0, -5) == qj.ERR_INVALID_ARGUMENT  # negative dither base
    assert call(1 << 20, 1 << 13, 1 << 13, 0) == qj.ERR_UNSUPPORTED  # 2^33 keys
    assert call(0, 2, 8, 0) == qj.OK and call(2, 0, 8, 8) == qj.OK  # nothing to write
    assert lib.qjl_quantize_keys_into(sk.handle, None, 1, 2, 2, 8, 0, 0, None, None, None) == \
        qj.ERR_INVALID_ARGUMENT
    sk.close()


@pytest.mark.parametrize("variant,d,m", [("dense", 128, 256), ("dense", 64, 512),
                                         ("dense", 128, 128), ("fqjl", 128, 256),
                                         ("fqjl", 128, 512), ("pfqjl", 128, 128),
                                         ("fqjl", 256, 512), ("pfqjl", 256, 256)])
def test_projected_keys_reproduce_their_bits(variant, d, m):
    # Projecting bf16 keys as queries applies the same sketch as quantizing
    # them (dense: the same bf16 S; FQJL: the same +-1 first stage, float32
    # matrix-core accumulation in the same order, the same second stage), so
    # the signs of the projection are the quantized bits, bit for bit.
    note("project-vs-quantize", variant, d, m)
    n = 333
    K = torch.randn(n, d, generator=torch.Generator().manual_seed(d + m)).to(torch.bfloat16)
    sk = qj.make_sketch(9, d, m, variant, 0.0)
    norms, bits = qj.quantize_keys(sk, K.to(DEV))
    Sq = qj.project_query(sk, K.to(DEV))
    torch.cuda.synchronize()
    got = oq.unpack_bits(bits_np(bits), m).astype(bool)
    want = to_np_f64(Sq) >= 0
    assert got.shape == want.shape and np.array_equal(got, want)
    sk.close()


@pytest.mark.parametrize("m,G,nq,nk", [(256, 1, 16, 4096), (256, 3, 1, 1000), (512, 2, 1, 777),
                                       (32, 2, 3, 65), (96, 1, 2, 130), (1024, 1, 1, 300),
                                       (128, 5, 4, 17), (256, 2, 7, 1), (2048, 1, 2, 64),
                                       (1024, 2, 3, 300), (1024, 1, 4, 5000),
                                       # at least a group per compute unit: each group
                                       # split into up to four parts, the last one short
                                       (256, 300, 1, 1000), (256, 256, 3, 2500),
                                       (512, 260, 2, 777), (128, 256, 1, 4097)])
def test_score_random_bits(m, G, nq, nk):
    # m = 1024 with query pairs: the kernel whose stage ring and query image
    # leave the least LDS for deferred scores (and no room for the default
    # 64 KB allowance) still defers them.
    note("score", m, G, nq, nk)
    rs = np.random.default_rng(m + G + nq + nk)
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    bits = wl.make_random_bits(G * nk, m, seed=7).to(DEV)
    norms = torch.from_numpy(np.abs(rs.standard_normal(G * nk)).astype(np.float32) * 10).to(DEV)
    Sq = torch.from_numpy((rs.standard_normal((G * nq, m)) * 11).astype(np.float32)).to(DEV)
    out = qj.score(sk, Sq, bits, norms, G, nq, nk)
    torch.cuda.synchronize()
    ref = oq.score(to_np_f64(Sq), bits_np(bits), to_np_f64(norms), m, 0.0, G, nq, nk)
    check_scores(to_np_f64(out), ref)
    sk.close()


@pytest.mark.parametrize("m,nq", [(256, 1), (512, 1), (1024, 3), (256, 6)])
def test_score_query_edge_values(m, nq):
    # The query becomes integers X_j = rint(Sq_j 2^F) with F set by its
    # largest |Sq_j|: a zero query (F = 0, every score exactly 0), a query
    # whose one large coordinate sets F, queries near the float32 denormal
    # range and signed zeros, against the oracle on the same bits and norms.
    note("score edge queries", m, nq)
    G, nk = 3, 777
    rs = np.random.default_rng(m + nq)
    sk = qj.make_sketch(0, 128, m, "dense", 0.0)
    bits = wl.make_random_bits(G * nk, m, seed=11).to(DEV)
    norms = torch.from_numpy(np.abs(rs.standard_normal(G * nk)).astype(np.float32) * 10).to(DEV)
    Sq = (rs.standard_normal((G * nq, m)) * 11).astype(np.float32)
    Sq[0] = 0.0                                   # a zero query
    Sq[1, :] = 1e-3
    Sq[1, 7] = 3e7                                # one coordinate sets the exponent
    Sq[2] = (rs.standard_normal(m) * 1e-36).astype(np.float32)   # tiny
    if nq > 1:
        Sq[3] = np.where(rs.random(m) < 0.5, -0.0, 0.0).astype(np.float32)  # signed zeros
    Sqd = torch.from_numpy(Sq).to(DEV)
    out = qj.score(sk, Sqd, bits, norms, G, nq, nk)
    torch.cuda.synchronize()
    ref = oq.score(to_np_f64(Sqd), bits_np(bits), to_np_f64(norms), m, 0.0, G, nq, nk)
    got = to_np_f64(out)
    check_scores(got, ref)
    assert np.all(got[0, 0] == 0.0)
    if nq > 1:
        assert np.all(got[3 // nq, 3 % nq] == 0.0)   # query row 3: signed zeros
    sk.close()


@pytest.mark.parametrize("variant,d,m,dt,rho", [
    ("dense", 512, 64, "bf16", 0.0),      # largest dense d
    ("dense", 1, 32, "f32", 0.0),         # smallest d and m
    ("dense", 128, 8192, "bf16", 0.0),    # largest m
    ("dense", 64, 8192, "f32", 0.2),
    ("fqjl", 128, 8192, "bf16", 0.1),     # 64 stacked blocks
    ("fqjl", 8, 8192, "f32", 0.0),
    ("dfqjl", 128, 8192, "bf16", 0.1),
    ("pfqjl", 16, 8192, "f32", 0.0),
])
def test_size_limits(variant, d, m, dt, rho):
    w = wl.Workload(f"limit_{variant}_{d}_{m}", d, m, variant, 1, 3, 67, 3, dt, "normal", rho,
                    seed=9)
    note("limits", variant, d, m, dt, rho)
    _, K, bits, norms, rb, rn = run_quantize_case(w)
    q = wl.make_queries(w, "cpu").to(DEV)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Sq = qj.project_query(sk, q)
    out = qj.score(sk, Sq, bits, norms, w.groups, w.n_q, w.n_k)
    torch.cuda.synchronize()
    ref = oracle_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Sq_ref = oq.project(ref, to_np_f64(q), w.dtype)
    check_projection(to_np_f64(Sq), Sq_ref, to_np_f64(q), w.m)
    s_ref = oq.score(Sq_ref, rb, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    slack = inband_slack(bits_np(bits), rb, Sq_ref, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    # the GPU scores its own projected query: widen by the projection's
    # difference, which moves a score by at most c ||k|| sum_j |dSq_j|
    dsq = np.abs(to_np_f64(Sq) - Sq_ref).sum(axis=1).reshape(w.groups, w.n_q, 1)
    c = oq.estimator_constant(w.m, w.rho)
    slack = slack + c * rn.reshape(w.groups, 1, w.n_k) * dsq
    check_scores(to_np_f64(out), s_ref, slack)
    sk.close()


def test_one_sketch_two_streams_concurrently():
    # a sketch is immutable: two streams quantizing and scoring different
    # caches with it at once give each the results it gets alone
    note("two streams")
    w = wl.DECODE_7B.scaled(batch=1, heads=8, n_k=4096)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant)
    K1 = wl.make_keys(w, DEV)
    K2 = (K1.float() * -0.5 + 0.25).to(torch.bfloat16)
    q = wl.make_queries(w, DEV)
    ref = []
    for K in (K1, K2):
        n, b = qj.quantize_keys(sk, K)
        Sq = qj.project_query(sk, q)
        ref.append((n, b, qj.score(sk, Sq, b, n, w.groups, w.n_q, w.n_k)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    torch.cuda.synchronize()
    for _ in range(3):
        outs.clear()
        for K, st in zip((K1, K2), streams):
            with torch.cuda.stream(st):
                n, b = qj.quantize_keys(sk, K, stream=st)
                Sq = qj.project_query(sk, q, stream=st)
                outs.append((n, b, qj.score(sk, Sq, b, n, w.groups, w.n_q, w.n_k, stream=st)))
        torch.cuda.synchronize()
        for (n, b, s), (rn, rb, rs) in zip(outs, ref):
            assert torch.equal(b, rb) and torch.equal(n, rn) and torch.equal(s, rs)
    sk.close()


def test_score_dither_constant():
    # rho enters the score only through sqrt(1 + rho^2)
    m, G, nq, nk = 256, 1, 2, 300
    rs = np.random.default_rng(1)
    sk = qj.make_sketch(0, 128, m, "fqjl", 0.7)
    bits = wl.make_random_bits(G * nk, m, seed=9).to(DEV)
    norms = torch.ones(G * nk, device=DEV)
    Sq = torch.from_numpy(rs.standard_normal((nq, m)).astype(np.float32)).to(DEV)
    out = qj.score(sk, Sq, bits, norms, G, nq, nk)
    ref = oq.score(to_np_f64(Sq), bits_np(bits), to_np_f64(norms), m, 0.7, G, nq, nk)
    check_scores(to_np_f64(out), ref)


@pytest.mark.parametrize("w", [wl.TINY, wl.DECODE_7B.scaled(batch=1, heads=2, n_k=999),
                               wl.FQJL_7B_DITHER.scaled(batch=1, heads=2, n_k=500),
                               wl.DFQJL_7B.scaled(batch=1, heads=2, n_k=500),
                               wl.PFQJL_7B.scaled(batch=1, heads=2, n_k=500)],
                         ids=lambda w: w.name)
def test_end_to_end_scores(w):
    note("e2e", w.name)
    _, K, bits, norms, rb, rn = run_quantize_case(w)
    q = wl.make_queries(w, "cpu").to(DEV)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Sq = qj.project_query(sk, q)
    out = qj.score(sk, Sq, bits, norms, w.groups, w.n_q, w.n_k)
    torch.cuda.synchronize()
    ref = oracle_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Sq_ref = oq.project(ref, to_np_f64(q), w.dtype)
    # the oracle's own bits and norms; in-band sign differences widen the bound
    s_ref = oq.score(Sq_ref, rb, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    slack = inband_slack(bits_np(bits), rb, Sq_ref, rn, w.m, w.rho, w.groups, w.n_q, w.n_k)
    check_scores(to_np_f64(out), s_ref, slack)
    sk.close()


@pytest.mark.parametrize("variant,rho,n", [("dense", 0.0, 300), ("dense", 0.0, 20000),
                                           ("dense", 0.3, 300), ("fqjl", 0.2, 300),
                                           ("fqjl", 0.2, 20000), ("dfqjl", 0.1, 300)])
def test_power_of_two_scaling_is_exact(variant, rho, n):
    # Scaling bf16 keys by 2^e is exact and commutes with every float32
    # product, sum and square root of the path (and the dither scales with
    # the norm), so the bits are identical and the norms scale by exactly
    # 2^e; scaling the projected queries scales every score by exactly 2^e.
    note("power-of-two scaling", variant, rho, n)
    d, m = 128, 256
    gen = torch.Generator().manual_seed(n + int(rho * 10))
    K = (torch.randn(n, d, generator=gen) * 3).to(torch.bfloat16).to(DEV)
    sk = qj.make_sketch(13, d, m, variant, rho)
    n0, b0 = qj.quantize_keys(sk, K, key_index_base=21)
    q = (torch.randn(4, d, generator=gen)).to(torch.bfloat16).to(DEV)
    Sq = qj.project_query(sk, q)
    s0 = qj.score(sk, Sq, b0, n0, 1, 4, n)
    for e in (50, -50):
        f = 2.0 ** e
        n1, b1 = qj.quantize_keys(sk, (K.float() * f).to(torch.bfloat16), key_index_base=21)
        s1 = qj.score(sk, Sq * f, b0, n0, 1, 4, n)
        torch.cuda.synchronize()
        assert torch.equal(b1, b0), e
        assert torch.equal(n1, n0 * f), e
        assert torch.equal(s1, s0 * f), e
    sk.close()


@pytest.mark.parametrize("variant,n", [("dense", 300), ("dense", 20000), ("fqjl", 300),
                                       ("fqjl", 20000), ("pfqjl", 300)])
def test_negated_keys_complement_every_bit(variant, n):
    # Without dither, negating a key negates every product and sum exactly,
    # so each coordinate changes sign (none is exactly zero for these keys):
    # the bits of -k are the complement of those of k, the norms are equal.
    note("negated keys", variant, n)
    gen = torch.Generator().manual_seed(n + 5)
    K = (torch.randn(n, 128, generator=gen) * 3).to(torch.bfloat16).to(DEV)
    sk = qj.make_sketch(17, 128, 256, variant, 0.0)
    n0, b0 = qj.quantize_keys(sk, K)
    n1, b1 = qj.quantize_keys(sk, -K)
    torch.cuda.synchronize()
    assert torch.equal(b1, ~b0)
    assert torch.equal(n1, n0)
    sk.close()


def test_zero_key_and_empty_calls():
    note("edge zero/empty")
    for variant, dt in (("dense", torch.float32), ("dense", torch.bfloat16), ("fqjl", torch.bfloat16)):
        sk = qj.make_sketch(0, 128, 256, variant, 0.2)
        K = torch.zeros(70, 128, dtype=dt, device=DEV)
        norms, bits = qj.quantize_keys(sk, K)
        torch.cuda.synchronize()
        assert np.all(bits_np(bits) == 0xFFFFFFFF)
        assert float(norms.abs().max()) == 0.0
        Sq = qj.project_query(sk, torch.randn(1, 128, device=DEV).to(dt))
        s = qj.score(sk, Sq, bits, norms, 1, 1, 70)
        torch.cuda.synchronize()
        assert float(s.abs().max()) == 0.0
        lib = qj.load()
        assert lib.qjl_quantize_keys(sk.handle, None, 1, 0, 0, None, None, None) == 0
        assert lib.qjl_project_query(sk.handle, None, 1, 0, None, None) == 0
        assert lib.qjl_score(sk.handle, None, None, None, 0, 1, 1, None, None) == 0
        assert lib.qjl_score(sk.handle, None, None, None, 1, 1, 0, None, None) == 0
        sk.close()


def test_invalid_arguments_on_gpu():
    note("edge invalid")
    sk = qj.make_sketch(0, 128, 256, "dense")
    lib = qj.load()
    K = torch.zeros(8, 128, dtype=torch.bfloat16, device=DEV)
    nrm = torch.zeros(8, device=DEV)
    bits = torch.zeros(8, 8, dtype=torch.int32, device=DEV)
    p = K.data_ptr()
    assert lib.qjl_quantize_keys(sk.handle, p + 1, 1, 8, 0, nrm.data_ptr(), bits.data_ptr(), None) == 1
    assert lib.qjl_quantize_keys(sk.handle, p, 5, 8, 0, nrm.data_ptr(), bits.data_ptr(), None) == 1
    assert lib.qjl_quantize_keys(sk.handle, p, 1, -1, 0, nrm.data_ptr(), bits.data_ptr(), None) == 1
    assert lib.qjl_quantize_keys(sk.handle, p, 1, 8, -5, nrm.data_ptr(), bits.data_ptr(), None) == 1
    assert lib.qjl_quantize_keys(sk.handle, p, 1, 8, 0, nrm.data_ptr() + 2, bits.data_ptr(), None) == 1
    assert lib.qjl_score(sk.handle, nrm.data_ptr(), bits.data_ptr(), nrm.data_ptr(), 1, -1, 1,
                         nrm.data_ptr(), None) == 1
    sk.close()
    assert sk._h.value is None


def test_sketch_export_matches_oracle():
    note("export")
    for (d, m) in ((128, 256), (128, 512), (100, 64)):
        sk = qj.make_sketch(0, d, m, "dense")
        s32, s16 = qj.sketch_export(sk, bf16=True)
        ref = oracle_sketch(0, d, m, "dense", 0.0)
        assert np.array_equal(s32.astype(np.float64), ref.S32)
        assert np.array_equal(s16, osk.bf16_bits(ref.S16))
        assert sk.info()["device"] == 0
        sk.close()
    for (d, m) in ((128, 256), (16, 64)):
        sk = qj.make_sketch(0, d, m, "fqjl")
        s32, _ = qj.sketch_export(sk)
        E = oracle_sketch(0, d, m, "fqjl", 0.0).explicit()
        assert np.allclose(s32, E, rtol=1e-6, atol=1e-6 * np.abs(E).max())
        sk.close()


def test_dither_key_index_base_appends():
    note("dither base")
    w = wl.FQJL_7B_DITHER.scaled(batch=1, heads=1, n_k=300)
    K = wl.make_keys(w, "cpu").to(DEV)
    sk = qj.make_sketch(0, 128, 256, "fqjl", 0.1)
    _, whole = qj.quantize_keys(sk, K, key_index_base=1000)
    _, a = qj.quantize_keys(sk, K[:123].contiguous(), key_index_base=1000)
    _, b = qj.quantize_keys(sk, K[123:].contiguous(), key_index_base=1123)
    torch.cuda.synchronize()
    assert torch.equal(whole, torch.cat([a, b]))
    sk.close()


# ---------------------------------------------------------------- full size
# The full-size workloads run in the launch configuration the benchmark
# times, and every output is compared with the oracle: all rows' bits and
# norms, every group's scores (the oracle runs chunk by chunk on a thread
# pool of the host's cores).
def full_size_quantize(w: wl.Workload):
    note("full quantize", w.name)
    K = wl.make_keys(w, DEV)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms, bits = qj.quantize_keys(sk, K)
    torch.cuda.synchronize()
    ref = oracle_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    Kh = K.cpu()
    nband, rb, rn = oracle_check_all_rows(ref, Kh, w.dtype, bits_np(bits), to_np_f64(norms))
    note("in-band sign differences, all rows:", nband)
    report_inband(f"{w.name} (all {w.n_keys} keys)", w.n_keys * w.m, nband)
    return sk, ref, norms, bits, rb, rn


def full_size_score(w: wl.Workload, sk, ref, norms, bits, rb, rn):
    note("full score", w.name)
    q = wl.make_queries(w, DEV)
    Sq = qj.project_query(sk, q)
    # the GPU scores its own bits and norms; the oracle scores its own
    out = qj.score(sk, Sq, bits, norms, w.groups, w.n_q, w.n_k)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    oracle_check_all_scores(ref, q.cpu(), w.dtype, to_np_f64(Sq), to_np_f64(out), bits_np(bits),
                            rb, rn, w.rho, w.groups, w.n_q, w.n_k)


def _full(w: wl.Workload, scores: bool):
    sk, ref, norms, bits, rb, rn = full_size_quantize(w)
    if scores:
        full_size_score(w, sk, ref, norms, bits, rb, rn)
    sk.close()


def test_full_size_decode_7b():
    _full(wl.DECODE_7B, scores=True)


def test_full_size_long_context():
    _full(wl.LONG_CTX, scores=True)


def test_full_size_prefill():
    _full(wl.PREFILL, scores=False)


@pytest.mark.parametrize("w", [wl.FQJL_7B, wl.FQJL_7B_DITHER, wl.DFQJL_7B], ids=lambda w: w.name)
def test_full_size_fqjl(w):
    _full(w, scores=True)


@pytest.mark.parametrize("variant", ["dense", "fqjl"])
def test_buffers_past_4gb(variant):
    # 2^26 + 4173 bf16 keys at d = 128, m = 512: the keys take 17 GB and the
    # bits 4.3 GB, so the last rows sit past byte offset 2^32 in both, and
    # one query scored against every key (a single group) writes 268 MB of
    # scores.  The first, the last and randomly chosen rows (bits, norms and
    # scores) are checked against the oracle.
    n, d, m = (1 << 26) + 4173, 128, 512
    note("buffers past 4 GB", variant, n)
    gen = torch.Generator(device=DEV).manual_seed(31)
    K = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    step = 1 << 22
    for i in range(0, n, step):
        j = min(n, i + step)
        K[i:j] = torch.randn(j - i, d, generator=gen, device=DEV).to(torch.bfloat16)
    q = torch.randn(1, d, generator=gen, device=DEV).to(torch.bfloat16)
    sk = qj.make_sketch(0, d, m, variant, 0.0)
    norms, bits = qj.quantize_keys(sk, K)
    Sq = qj.project_query(sk, q)
    s = qj.score(sk, Sq, bits, norms, 1, 1, n)
    torch.cuda.synchronize()
    pick = np.random.default_rng(5).choice(n, 1500, replace=False)
    rows = np.unique(np.concatenate([np.arange(300), np.arange(n - 300, n), pick]))
    assert rows[-1] * (m // 8) >= (1 << 32)  # the checked rows include bits past 4 GB
    idx = torch.from_numpy(rows).to(DEV)
    Kh = K.index_select(0, idx).cpu()
    gb = bits_np(bits.index_select(0, idx))
    gn = to_np_f64(norms.index_select(0, idx))
    gs = to_np_f64(s.reshape(-1).index_select(0, idx)).reshape(1, 1, -1)
    del K, bits, norms, s
    torch.cuda.empty_cache()
    ref = oracle_sketch(0, d, m, variant, 0.0)
    rb, rn, mg, _ = oq.quantize(ref, to_np_f64(Kh), "bf16")
    nband = check_bits(gb, rb, mg, m)
    check_norms(gn, rn)
    Sq_ref = oq.project(ref, to_np_f64(q.cpu()), "bf16")
    k = len(rows)
    s_ref = oq.score(Sq_ref, rb, rn, m, 0.0, 1, 1, k)
    check_scores(gs, s_ref, inband_slack(gb, rb, Sq_ref, rn, m, 0.0, 1, 1, k))
    report_inband(f"{variant}_n{n}_m{m} ({k} sampled keys; bits and keys past 4 GB)", k * m, nband)
    sk.close()
