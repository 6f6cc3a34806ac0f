"""The allocation-free decode attention (qjl_decode_attention_noalloc)
against qjl_decode_attention with a caller workspace: identical outputs on
two calls in a row, the second smaller, for the fused paths (one query,
multi-query) and the plain path (scores in the scratch), and the size
limit rejected before any launch."""
from __future__ import annotations

import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import bit_quantized_jl_amd as qj
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def _inputs(G, nq, nk, m, d_v, vdt, seed):
    rs = np.random.default_rng(seed)
    bits = wl.make_random_bits(G * nk, m, seed=seed).to(DEV)
    norms = torch.from_numpy(np.abs(rs.standard_normal(G * nk)).astype(np.float32) * 4).to(DEV)
    Sq = torch.from_numpy((rs.standard_normal((G * nq, m)) * 11).astype(np.float32)).to(DEV)
    V = torch.from_numpy(rs.standard_normal((G * nk, d_v)).astype(np.float32)).to(vdt).to(DEV)
    return Sq, bits, norms, V


@pytest.mark.parametrize("m,d_v,vdt,big,small", [
    (256, 128, torch.bfloat16, (32, 1, 20000), (8, 1, 3001)),    # fused, partials + combine
    (256, 128, torch.bfloat16, (300, 1, 2048), (4, 2, 999)),     # a group per workgroup
    (512, 128, torch.bfloat16, (16, 4, 8192), (3, 3, 513)),      # multi-query, matrix-core sums
    (256, 64, torch.float32, (8, 2, 4096), (2, 1, 77)),          # plain path: scores in scratch
])
def test_noalloc_matches_workspace_entry_point(m, d_v, vdt, big, small):
    sk = qj.make_sketch(0, 128, m, "dense")
    scale = 1.0 / math.sqrt(128)
    for i, (G, nq, nk) in enumerate((big, small)):
        note("noalloc", m, d_v, vdt, G, nq, nk)
        Sq, bits, norms, V = _inputs(G, nq, nk, m, d_v, vdt, seed=10 * i + m)
        need = qj.decode_attention_workspace_size(sk, G, nq, nk, d_v)
        assert need <= qj.NOALLOC_SCRATCH_BYTES
        ref = qj.decode_attention(sk, Sq, bits, norms, V, G, nq, nk, scale)
        out = torch.full((G, nq, d_v), float("nan"), device=DEV)
        qj.decode_attention_noalloc(sk, Sq, bits, norms, V, G, nq, nk, scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), float((out - ref).abs().max())
    sk.close()


def test_noalloc_rejects_oversized_workspace():
    # The plain path (d_v != 128) keeps every score in the workspace:
    # 1 x 1 x 9,000,000 keys need 36 MB > 32 MiB.  Rejected before any
    # launch, so the (tiny) buffers are never read.
    note("noalloc size limit")
    sk = qj.make_sketch(0, 128, 256, "dense")
    nk = 9_000_000
    assert qj.decode_attention_workspace_size(sk, 1, 1, nk, 64) > qj.NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1024, dtype=torch.float32, device=DEV)
    p = buf.data_ptr()
    lib = qj.load()
    st = lib.qjl_decode_attention_noalloc(sk.handle, p, p, p, p, qj.DTYPE_F32, 64, 1, 1, nk,
                                          1.0, p, None)
    assert st == qj.ERR_UNSUPPORTED
    # and a no-op call with no groups touches nothing
    assert lib.qjl_decode_attention_noalloc(sk.handle, None, None, None, None, 1, 128, 0, 1, 1,
                                            1.0, None, None) == qj.OK
    torch.cuda.synchronize()
    sk.close()
