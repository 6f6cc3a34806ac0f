"""The per-token decode step (append new keys, project new queries, fused
attention over the cache) captured into a HIP graph and replayed.

Every hot entry point only enqueues kernels on the caller's stream (no
allocation, copy, memset or synchronisation), so a caller can capture a
decode step once and replay it per token.  Each replay here runs on fresh
inputs written in place between replays, with eager library calls and
synchronisations in between, and must reproduce the eager call on the same
inputs exactly (same kernels, same launch shapes, fixed reduction orders).
The eager path itself is checked against the oracle in the other GPU tests.
"""
from __future__ import annotations

import math
import sys

import pytest
import torch

import bit_quantized_jl_amd as qj
import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("variant,G,nq,nk", [("dense", 32, 1, 2048), ("fqjl", 16, 1, 1000),
                                             ("dense", 8, 4, 3000)])
def test_decode_step_graph_replays_match_eager(variant, G, nq, nk):
    note("graph decode step", variant, G, nq, nk)
    d, m, dv = 128, 256, 128
    sk = qj.make_sketch(11, d, m, variant, 0.0)
    gen = torch.Generator().manual_seed(G * 1000 + nq * 10 + nk)

    def fresh(shape, dtype=torch.bfloat16, scale=1.0):
        return (torch.randn(*shape, generator=gen) * scale).to(dtype)

    # the cache (resident) and the step's inputs and outputs, all allocated up front
    bits = wl.make_random_bits(G * nk, m, seed=41, device=DEV)
    norms = (torch.rand(G * nk, generator=gen) * 10 + 1).to(DEV)
    V = fresh((G * nk, dv)).to(DEV)
    Knew = fresh((G, d)).to(DEV)
    q = fresh((G * nq, d)).to(DEV)
    nb = torch.empty(G, dtype=torch.float32, device=DEV)
    bb = torch.empty((G, m // 32), dtype=torch.int32, device=DEV)
    Sq = torch.empty((G * nq, m), dtype=torch.float32, device=DEV)
    att = torch.empty(G, nq, dv, device=DEV)
    ws = torch.empty(qj.decode_attention_workspace_size(sk, G, nq, nk, dv), dtype=torch.uint8,
                     device=DEV)
    scale = 1.0 / math.sqrt(d)

    def step(st=None):
        qj.quantize_keys(sk, Knew, norms_out=nb, bits_out=bb, stream=st)
        qj.project_query(sk, q, Sq_out=Sq, stream=st)
        qj.decode_attention(sk, Sq, bits, norms, V, G, nq, nk, scale, workspace=ws, out=att,
                            stream=st)

    step()  # eager warm-up: first-call set-up happens outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    other = fresh((500, d)).to(DEV)
    for r in range(4):
        Knew.copy_(fresh((G, d)))
        q.copy_(fresh((G * nq, d)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (nb, bb, Sq, att)]
        qj.quantize_keys(sk, other)  # unrelated eager work between replays
        step()
        torch.cuda.synchronize()
        for name, g_t, e_t in zip(("norms", "bits", "Sq", "attention"), got, (nb, bb, Sq, att)):
            assert torch.equal(g_t, e_t), f"replay {r}: {name} differs from the eager call"
        assert torch.isfinite(att).all()
    sk.close()
