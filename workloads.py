"""Seeded synthetic inputs shaped like LLM key/query caches.

This module only draws random tensors.  It holds none of the sketch,
quantizer or estimator arithmetic, so both the HIP path and the CPU oracle
can be fed from it without sharing any of the method's code.

The shapes follow the key/value-cache setting that the QJL abstract (Majid
Daliri's scholarfeed page) and the KIVI abstract (Braverman's catalyzex page)
describe: keys of Llama-2-7B-like models (32 heads, head dimension 128), with
per-channel outliers, which KIVI reports for keys.  No dataset or weights are
used; these tensors stand in for real caches.

Seeds: keys 1, queries 2, outlier channels 3, Student-t channel scales 4,
values 5.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_KEYS = 1
SEED_QUERIES = 2
SEED_OUTLIERS = 3
SEED_TSCALE = 4
SEED_VALUES = 5


@dataclass(frozen=True)
class Workload:
    """One named workload: sketch parameters plus the input recipe."""

    name: str
    d: int
    m: int
    variant: str            # "dense" | "fqjl" | "dfqjl" | "pfqjl"
    batch: int
    heads: int
    n_k: int                # keys per (batch, head)
    n_q: int                # queries per (batch, head)
    dtype: str              # "f32" | "bf16"
    keys: str = "normal"    # "normal" | "outliers" | "tscale"
    rho: float = 0.0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def groups(self) -> int:
        return self.batch * self.heads

    @property
    def n_keys(self) -> int:
        return self.groups * self.n_k

    @property
    def n_queries(self) -> int:
        return self.groups * self.n_q

    def scaled(self, **kw) -> "Workload":
        """Same recipe at another size (for oracle-sized parity runs)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads.  Sizes are the full ones; tests scale n_k / batch down
# where the CPU oracle must see every output.
TINY = Workload("tiny_single_head_d128_m256_n4096_q16", 128, 256, "dense",
                1, 1, 4096, 16, "f32", "normal")
DECODE_7B = Workload("llama7b_decode_b8_h32_ctx8192_m256", 128, 256, "dense",
                     8, 32, 8192, 1, "bf16", "outliers")
LONG_CTX = Workload("long_context_b1_h32_ctx131072_m512", 128, 512, "dense",
                    1, 32, 131072, 1, "bf16", "normal")
PREFILL = Workload("prefill_b16_h32_keys4096_m256", 128, 256, "dense",
                   16, 32, 4096, 1, "bf16", "tscale")
FQJL_7B = Workload("fqjl_llama7b_decode_b8_h32_ctx8192_m256", 128, 256, "fqjl",
                   8, 32, 8192, 1, "bf16", "outliers")
FQJL_7B_DITHER = FQJL_7B.scaled(name="fqjl_dither0.1_llama7b_decode_b8_h32_ctx8192_m256",
                                rho=0.1)

# the FQJL page's two constructions alone, on the same cache
DFQJL_7B = FQJL_7B.scaled(name="dfqjl_dither0.1_llama7b_decode_b8_h32_ctx8192_m256",
                          variant="dfqjl", rho=0.1)
PFQJL_7B = FQJL_7B.scaled(name="pfqjl_llama7b_decode_b8_h32_ctx8192_m256", variant="pfqjl")

ALL = [TINY, DECODE_7B, LONG_CTX, PREFILL, FQJL_7B, FQJL_7B_DITHER, DFQJL_7B, PFQJL_7B]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def channel_scales(w: Workload, device="cpu") -> torch.Tensor:
    """Per (head, channel) multipliers, shared over batch and tokens.

    "outliers": 4 distinct channels per head multiplied by 15.
    "tscale":   |t_3| (Student-t, 3 degrees of freedom) per (head, channel).
    "normal":   all ones.
    """
    s = torch.ones(w.heads, w.d, dtype=torch.float32, device=device)
    if w.keys == "outliers":
        g = _gen(SEED_OUTLIERS, "cpu")
        for h in range(w.heads):
            ch = torch.randperm(w.d, generator=g)[:4]
            s[h, ch.to(device)] = 15.0
    elif w.keys == "tscale":
        g = _gen(SEED_TSCALE, "cpu")
        z = torch.randn(w.heads, w.d, generator=g, dtype=torch.float64)
        chi = torch.randn(w.heads, w.d, 3, generator=g, dtype=torch.float64).pow(2).sum(-1)
        t3 = z / torch.sqrt(chi / 3.0)
        s = t3.abs().to(torch.float32).to(device)
    return s


def make_keys(w: Workload, device="cpu", n_k: int | None = None) -> torch.Tensor:
    """Keys as a [batch*heads*n_k, d] tensor in the workload dtype."""
    n_k = w.n_k if n_k is None else n_k
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    g = _gen(SEED_KEYS, device)
    out = torch.empty(w.batch, w.heads, n_k, w.d, dtype=dt, device=device)
    scales = channel_scales(w, device)
    # draw one (batch) slab at a time to bound the fp32 temporary
    for b in range(w.batch):
        x = torch.randn(w.heads, n_k, w.d, generator=g, dtype=torch.float32, device=device)
        if w.keys != "normal":
            x.mul_(scales[:, None, :])
        out[b].copy_(x.to(dt))
    return out.reshape(-1, w.d)


def make_queries(w: Workload, device="cpu") -> torch.Tensor:
    """Queries as a [batch*heads*n_q, d] tensor in the workload dtype."""
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    g = _gen(SEED_QUERIES, device)
    x = torch.randn(w.groups * w.n_q, w.d, generator=g, dtype=torch.float32, device=device)
    return x.to(dt)


def make_values(w: Workload, device="cpu", n_k: int | None = None, d_v: int | None = None,
                dtype: str = "bf16") -> torch.Tensor:
    """Cached value rows [batch*heads*n_k, d_v], standard normal, bf16 by
    default (the value cache is not sketched; d_v defaults to the head dim)."""
    n_k = w.n_k if n_k is None else n_k
    d_v = w.d if d_v is None else d_v
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = _gen(SEED_VALUES, device)
    out = torch.empty(w.groups, n_k, d_v, dtype=dt, device=device)
    for i in range(w.groups):
        out[i].copy_(torch.randn(n_k, d_v, generator=g, dtype=torch.float32, device=device).to(dt))
    return out.reshape(-1, d_v)


def make_random_bits(n_keys: int, m: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniformly random packed sign words [n_keys, m/32] (as int32 storage)."""
    g = _gen(seed, device)
    return torch.randint(-(2 ** 31), 2 ** 31, (n_keys, m // 32), generator=g,
                         dtype=torch.int64, device=device).to(torch.int32)
