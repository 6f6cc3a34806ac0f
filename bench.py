"""Benchmark: one step of the QJL hot path on the Llama-2-7B-shaped decode cache.

A step = quantize every key of the cache (batch 8 x 32 heads x 8192 tokens,
head_dim 128, dense m = 256 sketch, bf16 keys with per-channel outliers),
project the 256 queries (one per head), and score every (query, key) pair.
All inputs are synthetic (seeded) and already resident in HBM when the timed
region starts.

Printed (one JSON line): whole-step algorithmic throughput (GB/s), plus
  roofline      the dominant kernel (dense quantize), timed live with HIP
                events on the library's stream, against MI355X HBM peak;
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same step;
and extra per-kernel figures: keys quantized/s, the score kernel's GB/s on
caches rotated beyond the 256 MB Infinity Cache (cold) and on one cache that
stays in it (warm), the long-context (131072 tokens, m = 512) score, fused
decode attention, the other quantize configurations, the per-token decode
path, and each rate as a fraction of the 8 TB/s HBM peak, of the stream-copy
rate and of the plain read (and read-then-write) ceilings measured in the
same run.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QJL score GB/s (% of HBM peak) + keys quantized/s, 7B-shape decode"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PMC_SUMMARY = os.path.join(ROOT, "profiles", "quantize_dense_llama7b_decode_pmc.txt")
QUANT_KERNEL_SRC = os.path.join(ROOT, "bit_quantized_jl_amd", "csrc", "k_quantize_mfma.hip")
PROBE_LIB = os.path.join(ROOT, "bit_quantized_jl_amd", "libqjl_probe.so")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time for the oracle baseline sample")
    p.add_argument("--skip-extras", action="store_true",
                   help="only the timed step (used under profilers)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run only a plain 1 GiB device copy (reference for HBM byte counters)")
    p.add_argument("--only", choices=["quantize", "fqjl", "fqjl_dither", "score", "attention"],
                   help="run only a few launches of one kernel on its 7B-decode-shape workload "
                        "(for hardware-counter passes)")
    p.add_argument("--tu-hash", metavar="SOURCE",
                   help="print the hash of a kernel source and every header it includes "
                        "(the value recorded in profiles/*_pmc.txt) and exit")
    p.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                   help="run only the 7B-shape quantize launch (dense; with --only fqjl or "
                        "fqjl_dither the FQJL sketch) back to back for SECONDS while sampling "
                        "socket power and graphics clocks with amd-smi")
    return p.parse_args()


def calibrate_copy():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, the
    reference that scales rocprofv3's FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": a.numel() * 4,
                      "calibrate_copy_bytes_written": a.numel() * 4}), flush=True)


def sustain(seconds: float, kind: str | None = None):
    """A quantize kernel under sustained load: the 7B-shape quantize (dense, or
    with --only fqjl / fqjl_dither the FQJL sketch without or with dither)
    launched back to back for `seconds`, with amd-smi sampling socket power and
    the graphics clocks of every XCD in a child process meanwhile.  Prints one
    JSON line: mean launch time, mean power, mean clock (samples of the first
    second, while the clocks settle, are dropped)."""
    import re
    import subprocess
    import torch

    import bit_quantized_jl_amd as qj
    import workloads as wl

    qj.load()
    w = {None: wl.DECODE_7B, "quantize": wl.DECODE_7B, "fqjl": wl.FQJL_7B,
         "fqjl_dither": wl.FQJL_7B_DITHER}[kind]
    dev = "cuda:0"
    K = wl.make_keys(w, dev)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms = torch.empty(w.n_keys, dtype=torch.float32, device=dev)
    bits = torch.empty((w.n_keys, w.m // 32), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    for _ in range(10):
        qj.quantize_keys(sk, K, norms_out=norms, bits_out=bits, stream=st)
    torch.cuda.synchronize()
    n_samples = max(1, int(seconds / 0.5) - 2)
    sampler = subprocess.Popen(
        ["bash", "-c", f"sleep 1; for i in $(seq {n_samples}); do amd-smi metric -p -c; sleep 0.3; done"],
        stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    a, b = HipEvent(), HipEvent()
    launches = 0
    t0 = time.time()
    a.record(st)
    while time.time() - t0 < seconds:
        for _ in range(50):
            qj.quantize_keys(sk, K, norms_out=norms, bits_out=bits, stream=st)
        launches += 50
        torch.cuda.synchronize()
    b.record(st)
    torch.cuda.synchronize()
    out = sampler.communicate()[0]
    power = [float(x) for x in re.findall(r"SOCKET_POWER: (\d+(?:\.\d+)?)", out)]
    clocks, section = [], ""
    for line in out.splitlines():
        head = re.match(r"\s*(\w+):\s*$", line)
        if head:
            section = head.group(1)
            continue
        clk = re.match(r"\s*CLK: (\d+) MHz", line)
        if clk and section.startswith("GFX_"):  # graphics clock of one XCD
            clocks.append(float(clk.group(1)))
    print(json.dumps({"sustain_s": seconds, "workload": w.name, "sketch": w.variant, "rho": w.rho,
                      "dense_schedule": dense_schedule(),
                      "launches": launches,
                      "mean_launch_s": a.seconds_to(b) / launches,
                      "socket_power_w_mean": sum(power) / len(power) if power else None,
                      "socket_power_w_samples": len(power),
                      "gfx_clock_mhz_mean": sum(clocks) / len(clocks) if clocks else None,
                      "gfx_clock_samples": len(clocks)}), flush=True)


def translation_unit_files(src: str) -> list:
    """A source file and every header it includes with #include "...",
    recursively (each once, in the order first reached)."""
    import re
    seen, order = set(), []

    def visit(path):
        path = os.path.normpath(path)
        if path in seen or not os.path.exists(path):
            return
        seen.add(path)
        order.append(path)
        with open(path) as f:
            for inc in re.findall(r'^\s*#\s*include\s+"([^"]+)"', f.read(), flags=re.M):
                visit(os.path.join(os.path.dirname(path), inc))

    visit(src)
    return order


def kernel_tu_hash(src: str = QUANT_KERNEL_SRC) -> str:
    """sha256 (first 16 hex digits) over a kernel's whole translation unit:
    the source and every header it includes, each as (path relative to the
    repository, contents), so a change to any of them changes the hash."""
    h = hashlib.sha256()
    for path in translation_unit_files(src):
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


DENSE_SCHEDULES = ("default", "prefetch", "rt4", "immediate")
# The instantiation each schedule launches at the 7B decode shape (d = 128,
# m = 256): <D, M, WAVES, RT, R, DEFER, PF, MAPPED>, as kernel traces name it.
DENSE_KERNEL_7B = {
    "default": "quantize_mfma_kernel<128, 256, 4, 2, 4, true, false, false>",
    "prefetch": "quantize_mfma_kernel<128, 256, 4, 2, 2, true, true, false>",
    "rt4": "quantize_mfma_kernel<128, 256, 4, 4, 2, false, false, false>",
    "immediate": "quantize_mfma_kernel<128, 256, 4, 2, 4, false, false, false>",
}


def dense_schedule() -> str:
    """The dense quantizer's register schedule this process launches: the
    library reads QJL_DENSE_SCHEDULE, and any value other than the three
    alternatives means the default."""
    s = os.environ.get("QJL_DENSE_SCHEDULE", "default")
    return s if s in DENSE_SCHEDULES else "default"


def read_traffic():
    """HBM bytes per quantize launch from the committed rocprofv3 PMC summary,
    or None when absent, taken on another version of the kernel's
    translation unit (its source or any header it includes), or taken with
    another register schedule than this process launches."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    vals = {}
    for line in open(PMC_SUMMARY):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_tu_sha256_16") != kernel_tu_hash():
        return None
    if vals.get("dense_schedule", "default") != dense_schedule():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, K_dev, seconds: float):
    """The float64 oracle on the (batch, head) groups of the same step, one
    group after another (group g = its 8192 cached keys, copied from the
    GPU, and its query), until about `seconds` of CPU time; throughput in the
    metric's unit (GB/s)."""
    import numpy as np
    import torch

    import workloads as wl
    from oracle import qjl as oq
    from oracle import sketch as osk

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    sk = osk.make_dense(w.seed, w.d, w.m)
    Kh = K_dev.cpu()                                # the step's cache, on the host
    q = wl.make_queries(w, "cpu").double().numpy()  # the step's queries (same recipe)
    t0 = time.perf_counter()
    groups = 0
    while True:
        g = groups
        K = Kh[g * w.n_k:(g + 1) * w.n_k].double().numpy()
        bits, norms, _, _ = oq.quantize(sk, K, w.dtype, key_index_base=g * w.n_k)
        Sq = oq.project(sk, q[g * w.n_q:(g + 1) * w.n_q], w.dtype)
        oq.score(Sq, bits, norms, w.m, 0.0, 1, w.n_q, w.n_k)
        groups += 1
        el = time.perf_counter() - t0
        if el >= seconds or groups >= w.groups:
            break
    per_group_bytes = step_bytes(w) / w.groups
    return {"value": per_group_bytes * groups / el / 1e9, "unit": "GB/s",
            "cores": int(min(cores, blas_threads)),
            "host_cores": cores, "blas_threads": blas_threads, "kind": "oracle",
            "sample": f"groups 0..{groups - 1} ({groups} of {w.groups} distinct (batch, head) "
                      f"groups of the same step: {groups * w.n_k} cached keys copied from the "
                      f"GPU and their queries; quantize + project + score, float64 numpy), "
                      f"{el:.1f} s"}


def quantize_bytes(w) -> float:
    esz = 2 if w.dtype == "bf16" else 4
    return w.n_keys * (w.d * esz + w.m / 8 + 4)


def score_bytes(w) -> float:
    return (w.groups * w.n_k * (w.m / 8 + 4) + w.groups * w.n_q * w.n_k * 4
            + w.groups * w.n_q * w.m * 4)


def score_write_bytes(w) -> float:
    """The scores the score kernel writes (the rest of score_bytes is read)."""
    return w.groups * w.n_q * w.n_k * 4


def quantize_write_bytes(w) -> float:
    """The bits and norms the quantize kernel writes (the keys are read)."""
    return w.n_keys * (w.m / 8 + 4)


def project_bytes(w) -> float:
    esz = 2 if w.dtype == "bf16" else 4
    return w.n_queries * (w.d * esz + w.m * 4)


def attention_bytes(w, d_v: int = 128) -> float:
    """Keys' bits and norms, bf16 value rows, projected queries in, outputs out
    (the per-wave partials in the workspace, a few MB, are not counted)."""
    return (w.groups * w.n_k * (w.m / 8 + 4 + 2 * d_v)
            + w.groups * w.n_q * (w.m * 4 + d_v * 4))


def step_bytes(w) -> float:
    return quantize_bytes(w) + project_bytes(w) + score_bytes(w)


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    skips the system-scope cache write-back and invalidate that a default
    event performs, which would otherwise stall the GPU for several
    microseconds at every record inside the timed region.  Uses the HIP
    runtime already loaded by torch (the one the library's streams belong to)."""

    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("HIP runtime not loaded")
            lib = ctypes.CDLL(path)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = lib
        return cls._lib

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self.lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self.lib().hipEventRecord(self._ev, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def seconds_to(self, other: "HipEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = self.lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, other._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value / 1e3

    def __del__(self):
        if self._lib is not None and getattr(self, "_ev", None):
            self._lib.hipEventDestroy(self._ev)


def time_quantize(qj, torch, w, reps: int = 10):
    """One quantize configuration on its own: `reps` launches back to back
    between two HIP events after two warm-up launches; returns seconds per
    launch and the algorithmic bytes of one launch."""
    import workloads as wl
    dev = "cuda:0"
    K = wl.make_keys(w, dev)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms = torch.empty(w.n_keys, dtype=torch.float32, device=dev)
    bits = torch.empty((w.n_keys, w.m // 32), dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()
    for _ in range(2):
        qj.quantize_keys(sk, K, norms_out=norms, bits_out=bits, stream=st)
    torch.cuda.synchronize()
    a, b = HipEvent(), HipEvent()
    a.record(st)
    for _ in range(reps):
        qj.quantize_keys(sk, K, norms_out=norms, bits_out=bits, stream=st)
    b.record(st)
    torch.cuda.synchronize()
    t = a.seconds_to(b) / reps
    sk.close()
    del K, norms, bits
    torch.cuda.empty_cache()
    return t, quantize_bytes(w)


def copy_peak_gbps(torch, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Measured stream-copy rate: bytes read plus bytes written per second by
    torch's device copy of one `nbytes` buffer into another (both far larger
    than the 256 MB Infinity Cache), best of `reps` timed copies."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    evs = [(HipEvent(), HipEvent()) for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        dst.copy_(src)
        b.record(st)
    torch.cuda.synchronize()
    best = min(a.seconds_to(b) for a, b in evs)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / best / 1e9


def per_call_times(torch, call, iters: int) -> list:
    """Sorted seconds of `iters` calls, each between its own fence-free HIP
    event pair on the current stream, with Python's garbage collector off:
    a collection between a call's start event and its launch, with the queue
    drained, would be timed as part of that call."""
    import gc
    st = torch.cuda.current_stream()
    evs = [(HipEvent(), HipEvent()) for _ in range(iters)]
    was = gc.isenabled()
    gc.disable()
    try:
        for i in range(iters):
            evs[i][0].record(st)
            call(i)
            evs[i][1].record(st)
        torch.cuda.synchronize()
    finally:
        if was:
            gc.enable()
    return sorted(a.seconds_to(b) for a, b in evs)


def read_ceiling(torch, nbytes: int, n_sets: int, iters: int = 40):
    """Measured read-bandwidth ceiling for a kernel that streams `nbytes`:
    plain 16-byte-vector read kernels (libqjl_probe.so: chunked and
    grid-stride patterns, 2/4/8 loads in flight per lane, 1/2/4 workgroups of
    256 lanes per compute unit) over `n_sets` distinct buffers of that size
    in rotation (as the score timing rotates its inputs past the 256 MB
    Infinity Cache), timed like the kernels: median of per-call HIP-event
    times.  Returns the best configuration's rate."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.qjl_probe_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    n16 = (nbytes + 15) // 16
    bufs = [torch.full((n16 * 4,), 1.0, dtype=torch.float32, device="cuda:0")
            for _ in range(n_sets)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(4 * cus * 256, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    best = None
    per_pattern = {}
    for pattern in (0, 1):
        for unroll in (2, 4, 8):
            for wpc in (1, 2, 4):
                grid = cus * wpc

                def call(i):
                    rc = fn(bufs[i % n_sets].data_ptr(), n16 * 16, pattern, unroll, grid,
                            sink.data_ptr(), st.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"qjl_probe_read failed ({rc})")

                for i in range(2 * n_sets):
                    call(i)
                torch.cuda.synchronize()
                ts = per_call_times(torch, call, iters)
                med = ts[len(ts) // 2]
                key = "chunked" if pattern == 0 else "grid-stride"
                per_pattern[key] = min(per_pattern.get(key, med), med)
                if best is None or med < best["median_s"]:
                    best = {"median_s": med, "mean_s": sum(ts) / len(ts),
                            "GBps": n16 * 16 / med / 1e9,
                            "pattern": "chunked" if pattern == 0 else "grid-stride",
                            "loads_in_flight_per_lane": unroll, "workgroups_per_cu": wpc}
    del bufs, sink
    torch.cuda.empty_cache()
    best["bytes"] = n16 * 16
    best["rotation"] = f"{n_sets} buffers"
    best["best_GBps_by_pattern"] = {k: n16 * 16 / v / 1e9 for k, v in per_pattern.items()}
    best["frac_hbm"] = best["GBps"] / HBM_PEAK_GBPS
    return best


def read_write_ceiling(torch, read_bytes: int, write_bytes: int, n_sets: int, iters: int = 40):
    """Measured ceiling for a kernel that reads `read_bytes` and writes
    `write_bytes`: the plain read kernels of read_ceiling, each workgroup then
    writing its contiguous share of the output with 16-byte non-temporal
    stores (libqjl_probe.so), over `n_sets` rotated (input, output) pairs,
    timed the same way; the best of the same 18 configurations.  The rate is
    (read + write bytes) / median time."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    fn = lib.qjl_probe_read_write
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n16 = (read_bytes + 15) // 16
    m16 = (write_bytes + 15) // 16
    bufs = [(torch.full((n16 * 4,), 1.0, dtype=torch.float32, device="cuda:0"),
             torch.empty(m16 * 4, dtype=torch.float32, device="cuda:0")) for _ in range(n_sets)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream()
    best = None
    for pattern in (0, 1):
        for unroll in (2, 4, 8):
            for wpc in (1, 2, 4):
                grid = cus * wpc

                def call(i):
                    src, dst = bufs[i % n_sets]
                    rc = fn(src.data_ptr(), n16 * 16, dst.data_ptr(), m16 * 16, pattern, unroll,
                            grid, st.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"qjl_probe_read_write failed ({rc})")

                for i in range(2 * n_sets):
                    call(i)
                torch.cuda.synchronize()
                ts = per_call_times(torch, call, iters)
                med = ts[len(ts) // 2]
                if best is None or med < best["median_s"]:
                    best = {"median_s": med, "mean_s": sum(ts) / len(ts),
                            "GBps": (n16 + m16) * 16 / med / 1e9,
                            "pattern": ("chunked" if pattern == 0 else "grid-stride")
                                       + " reads, then each workgroup's share of the writes",
                            "loads_in_flight_per_lane": unroll, "workgroups_per_cu": wpc}
    del bufs
    torch.cuda.empty_cache()
    best["read_bytes"] = n16 * 16
    best["write_bytes"] = m16 * 16
    best["rotation"] = f"{n_sets} input/output pairs"
    best["frac_hbm"] = best["GBps"] / HBM_PEAK_GBPS
    return best


# Memory and fabric clocks fall while the GPU idles (set-up, a host copy):
# the first tens of calls after such a stretch ran ~8% slower.  Each rotating
# measurement therefore starts with ~30 ms of untimed calls.
WARM_S = 0.03


def warm_up(torch, call, n_sets: int, est_s: float):
    """Untimed calls before a rotating measurement: every input set twice and
    at least WARM_S of GPU time (est_s: a rough duration of one call)."""
    for i in range(max(2 * n_sets, int(WARM_S / est_s) + 1)):
        call(i)
    torch.cuda.synchronize()


def back_to_back_mean(torch, call, iters: int) -> float:
    """Mean seconds per call of `iters` calls enqueued back to back between one
    pair of events (launch gaps included), garbage collector off."""
    import gc
    st = torch.cuda.current_stream()
    a, b = HipEvent(), HipEvent()
    was = gc.isenabled()
    gc.disable()
    try:
        a.record(st)
        for i in range(iters):
            call(i)
        b.record(st)
        torch.cuda.synchronize()
    finally:
        if was:
            gc.enable()
    return a.seconds_to(b) / iters


def time_score_rotating(qj, torch, w, sk, n_sets: int, iters: int):
    """Score kernel alone over `n_sets` distinct (bits, norms, Sq) sets, so the
    working set exceeds the 256 MB Infinity Cache: mean, median, p10 and p90
    seconds of per-call event times, then the mean of the same number of
    calls back to back."""
    import workloads as wl
    dev = "cuda:0"
    sets = []
    for s in range(n_sets):
        bits = wl.make_random_bits(w.groups * w.n_k, w.m, seed=100 + s, device=dev)
        norms = torch.rand(w.groups * w.n_k, device=dev) * 10 + 1
        Sq = torch.randn(w.groups * w.n_q, w.m, device=dev) * 11
        out = torch.empty(w.groups, w.n_q, w.n_k, device=dev)
        sets.append((Sq, bits, norms, out))
    st = torch.cuda.current_stream()

    def call(i):
        Sq, bits, norms, out = sets[i % n_sets]
        qj.score(sk, Sq, bits, norms, w.groups, w.n_q, w.n_k, scores_out=out, stream=st)

    warm_up(torch, call, n_sets, score_bytes(w) / 5e12)
    ts = per_call_times(torch, call, iters)
    b2b = back_to_back_mean(torch, call, iters)
    del sets
    torch.cuda.empty_cache()
    pct = lambda p: ts[min(len(ts) - 1, int(p * len(ts)))]
    return sum(ts) / len(ts), ts[len(ts) // 2], pct(0.1), pct(0.9), b2b


def time_attention_rotating(qj, torch, w, sk, n_sets: int, iters: int, d_v: int = 128):
    """Fused decode attention alone over `n_sets` distinct (bits, norms, V, Sq)
    sets (each larger than the 256 MB Infinity Cache); returns mean, median,
    p10 and p90 seconds per call."""
    import math
    import workloads as wl
    dev = "cuda:0"
    sets = []
    for s in range(n_sets):
        bits = wl.make_random_bits(w.groups * w.n_k, w.m, seed=200 + s, device=dev)
        norms = torch.rand(w.groups * w.n_k, device=dev) * 10 + 1
        Sq = torch.randn(w.groups * w.n_q, w.m, device=dev) * 11
        V = torch.randn(w.groups * w.n_k, d_v, device=dev).to(torch.bfloat16)
        out = torch.empty(w.groups, w.n_q, d_v, device=dev)
        sets.append((Sq, bits, norms, V, out))
    ws = torch.empty(qj.decode_attention_workspace_size(sk, w.groups, w.n_q, w.n_k, d_v),
                     dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(w.d)
    st = torch.cuda.current_stream()

    def call(i):
        Sq, bits, norms, V, out = sets[i % n_sets]
        qj.decode_attention(sk, Sq, bits, norms, V, w.groups, w.n_q, w.n_k, scale,
                            workspace=ws, out=out, stream=st)

    warm_up(torch, call, n_sets, attention_bytes(w, d_v) / 5e12)
    ts = per_call_times(torch, call, iters)
    del sets, ws
    torch.cuda.empty_cache()
    pct = lambda p: ts[min(len(ts) - 1, int(p * len(ts)))]
    return sum(ts) / len(ts), ts[len(ts) // 2], pct(0.1), pct(0.9)


def time_calls(torch, fn, iters: int):
    """(mean seconds per call back to back, median of per-call event times)."""
    st = torch.cuda.current_stream()
    for _ in range(5):
        fn(st)
    torch.cuda.synchronize()
    a, b = HipEvent(), HipEvent()
    a.record(st)
    for _ in range(iters):
        fn(st)
    b.record(st)
    torch.cuda.synchronize()
    b2b = a.seconds_to(b) / iters
    evs = [(HipEvent(), HipEvent()) for _ in range(iters)]
    for e0, e1 in evs:
        e0.record(st)
        fn(st)
        e1.record(st)
    torch.cuda.synchronize()
    ts = sorted(e0.seconds_to(e1) for e0, e1 in evs)
    return b2b, ts[len(ts) // 2]


def decode_time_extras(qj, torch, w, sk):
    """The per-token path at the 7B decode shape: append one new key per
    (batch, head) (256 keys), project the 256 new queries, and the fused
    attention of each query over its head's 8192 cached keys; plus
    multi-query scoring (n_q queries per cached head reuse one pass over
    the bits)."""
    import math
    import workloads as wl
    dev = "cuda:0"
    out = {}
    G = w.groups
    one = w.scaled(n_k=1)
    Knew = wl.make_keys(one, dev)                      # [256, 128] bf16
    q = wl.make_queries(w, dev)
    nb = torch.empty(G, dtype=torch.float32, device=dev)
    bb = torch.empty((G, w.m // 32), dtype=torch.int32, device=dev)
    Sq = torch.empty((w.n_queries, w.m), dtype=torch.float32, device=dev)
    t_b2b, t_med = time_calls(torch, lambda st: qj.quantize_keys(sk, Knew, norms_out=nb,
                                                                  bits_out=bb, stream=st), 200)
    out["append_256_keys"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med,
                              "keys": G, "sketch": "dense m=256"}
    t_b2b, t_med = time_calls(torch, lambda st: qj.project_query(sk, q, Sq_out=Sq, stream=st), 200)
    out["project_256_queries"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med}
    skf = qj.make_sketch(w.seed, w.d, w.m, "fqjl")
    t_b2b, t_med = time_calls(torch, lambda st: qj.project_query(skf, q, Sq_out=Sq, stream=st), 200)
    out["project_256_queries_fqjl"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med}
    t_b2b, t_med = time_calls(torch, lambda st: qj.quantize_keys(skf, Knew, norms_out=nb,
                                                                  bits_out=bb, stream=st), 200)
    out["append_256_keys_fqjl"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med}
    skf.close()
    # the whole per-token step on a resident cache: append + project + attention
    bits = wl.make_random_bits(G * w.n_k, w.m, seed=300, device=dev)
    norms = torch.rand(G * w.n_k, device=dev) * 10 + 1
    V = torch.randn(G * w.n_k, 128, device=dev).to(torch.bfloat16)
    att = torch.empty(G, w.n_q, 128, device=dev)
    ws = torch.empty(qj.decode_attention_workspace_size(sk, G, w.n_q, w.n_k, 128),
                     dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(w.d)

    # each head's new key goes straight into its cache slot (the last of n_k rows)
    t_b2b, t_med = time_calls(torch, lambda st: qj.quantize_keys_into(
        sk, Knew, G, norms, bits, w.n_k, w.n_k - 1, stream=st), 200)
    out["append_256_keys_into_cache"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med,
                                         "keys": G, "cache_rows_per_head": w.n_k}

    def step(st):
        qj.quantize_keys_into(sk, Knew, G, norms, bits, w.n_k, w.n_k - 1, stream=st)
        qj.project_query(sk, q, Sq_out=Sq, stream=st)
        qj.decode_attention(sk, Sq, bits, norms, V, G, w.n_q, w.n_k, scale, workspace=ws,
                            out=att, stream=st)

    t_b2b, t_med = time_calls(torch, step, 50)
    out["decode_token_step"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med,
                                "what": "append 256 keys into their cache rows + project "
                                        "256 queries + fused attention over 256 x 8192 "
                                        "cached keys (bf16 V), the new keys included"}
    # the same step captured once into a HIP graph and replayed per token
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    t_b2b, t_med = time_calls(torch, lambda st: graph.replay(), 50)
    out["decode_token_step_graph"] = {"mean_s_back_to_back": t_b2b, "median_s": t_med,
                                      "what": "the decode_token_step launches replayed as one "
                                              "HIP graph"}
    del graph
    del V, ws, att
    # multi-query scoring: n_q queries per cached head (GQA-style)
    mq = {}
    for nq in (1, 2, 4, 8, 16):
        Sqm = torch.randn(G * nq, w.m, device=dev) * 11
        sc = torch.empty(G, nq, w.n_k, device=dev)
        t_b2b, t_med = time_calls(torch, lambda st: qj.score(sk, Sqm, bits, norms, G, nq, w.n_k,
                                                              scores_out=sc, stream=st), 50)
        nbytes = G * w.n_k * (w.m / 8 + 4) + G * nq * w.n_k * 4 + G * nq * w.m * 4
        mq[str(nq)] = {"median_s": t_med, "scores_per_s": G * nq * w.n_k / t_med,
                       "GBps": nbytes / t_med / 1e9}
        del Sqm, sc
    out["score_multiquery"] = mq
    del bits, norms
    torch.cuda.empty_cache()
    # fused attention with several queries per cached head (grouped-query)
    am = {}
    for G2, nq in ((256, 1), (256, 4), (64, 8)):
        w2 = w.scaled(batch=1, heads=G2, n_q=nq)
        t_mean, t_med, _, _ = time_attention_rotating(qj, torch, w2, sk, n_sets=2, iters=30)
        am[f"{G2}x{nq}"] = {"median_s": t_med, "queries": G2 * nq, "keys_per_group": w2.n_k,
                            "GBps": attention_bytes(w2) / t_med / 1e9}
    out["attention_multiquery"] = am
    torch.cuda.empty_cache()
    return out


def run_only(kind: str):
    """A few launches of one kernel (for rocprofv3 counter passes)."""
    import torch

    import bit_quantized_jl_amd as qj
    import workloads as wl
    if kind == "attention":
        w = wl.DECODE_7B
        sk = qj.make_sketch(w.seed, w.d, w.m, w.variant)
        t = time_attention_rotating(qj, torch, w, sk, n_sets=1, iters=5)[0]
    elif kind == "score":
        w = wl.DECODE_7B
        sk = qj.make_sketch(w.seed, w.d, w.m, w.variant)
        t = time_score_rotating(qj, torch, w, sk, n_sets=1, iters=5)[0]
    else:
        w = {"quantize": wl.DECODE_7B, "fqjl": wl.FQJL_7B, "fqjl_dither": wl.FQJL_7B_DITHER}[kind]
        sk = None
        t = time_quantize(qj, torch, w, reps=3)[0]
    if sk is not None:
        sk.close()
    out = {"only": kind, "workload": w.name, "mean_s": t}
    if kind == "quantize":
        out["dense_schedule"] = dense_schedule()
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.tu_hash:
        print(kernel_tu_hash(os.path.abspath(args.tu_hash)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the kernels work on one GPU's shard; see the sharding note in the design).",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sustain > 0:
        sustain(args.sustain, args.only)
        return
    if args.only:
        run_only(args.only)
        return
    import torch

    import bit_quantized_jl_amd as qj
    import workloads as wl

    qj.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    w = wl.DECODE_7B
    K = wl.make_keys(w, dev)
    # the oracle's copy of the keys, taken now: the copy leaves the GPU idle
    K_host = K.cpu() if not args.no_cpu_baseline else None
    q = wl.make_queries(w, dev)
    sk = qj.make_sketch(w.seed, w.d, w.m, w.variant, w.rho)
    norms = torch.empty(w.n_keys, dtype=torch.float32, device=dev)
    bits = torch.empty((w.n_keys, w.m // 32), dtype=torch.int32, device=dev)
    Sq = torch.empty((w.n_queries, w.m), dtype=torch.float32, device=dev)
    scores = torch.empty((w.groups, w.n_q, w.n_k), dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(st)
        qj.quantize_keys(sk, K, norms_out=norms, bits_out=bits, stream=st)
        if ev is not None:
            ev[1].record(st)
        qj.project_query(sk, q, Sq_out=Sq, stream=st)
        qj.score(sk, Sq, bits, norms, w.groups, w.n_q, w.n_k, scores_out=scores, stream=st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: K steps back to back on the library's stream, with a
    # fence-free HIP event pair around each quantize launch (HipEvent: a
    # default event would write back the caches at every record).  The
    # dominant kernel's launch duration is read from exactly the launches the
    # step time covers; the chip's clock falls within milliseconds of
    # sustained load, so a separate pass would see another clock.  The event
    # records stay inside the step time.
    # Python's garbage collector stays off while the steps are enqueued.
    import gc
    evs = [(HipEvent(), HipEvent()) for _ in range(args.steps)]
    t_start, t_end = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    gc.disable()
    t_start.record(st)
    for i in range(args.steps):
        step(evs[i])
    t_end.record(st)
    torch.cuda.synchronize()
    gc.enable()
    total_s = t_start.seconds_to(t_end)
    per_step = total_s / args.steps
    q_times = [a.seconds_to(b) for a, b in evs]
    q_step_avg = sum(q_times) / len(q_times)
    ps_avg = per_step - q_step_avg

    qbytes = quantize_bytes(w)
    q_flops = 2.0 * w.n_keys * w.d * w.m
    q_avg = q_step_avg
    achieved = qbytes / q_avg / 1e9
    traffic = read_traffic()
    result = {
        "metric": METRIC,
        "value": step_bytes(w) / per_step / 1e9,
        "unit": "GB/s",
        "value_is": "algorithmic bytes of one whole step (quantize 2,097,152 keys + project "
                    "256 queries + score 256 x 8192 pairs: "
                    f"{step_bytes(w):.0f} B) / its time, K steps back to back (a fence-free "
                    "event pair around each quantize launch inside them); the score "
                    "kernel's own GB/s and fraction of HBM are in score_decode7b",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "context": w.n_k,
                   "head_dim": w.d, "m": w.m, "sketch": w.variant, "queries_per_head": w.n_q,
                   "keys": "bf16 N(0,1), 4 outlier channels x15 per head"},
        "roofline": {"kernel": DENSE_KERNEL_7B[dense_schedule()], "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": qbytes, "avg_launch_s": q_avg,
                     "dense_schedule": dense_schedule(),
                     "timing": "HIP events around each quantize launch inside the timed K steps",
                     "launch_s_min": min(q_times), "launch_s_max": max(q_times),
                     "mfma_tflops": q_flops / q_avg / 1e12,
                     "mfma_frac_bf16": q_flops / q_avg / 1e12 / BF16_PEAK_TFLOPS},
        "keys_quantized_per_s": w.n_keys / q_avg,
        "project_plus_score_s_approx": ps_avg,
    }
    if not args.skip_extras:
        # The kernels are timed before the probes (device copy, read ceilings):
        # those allocate and free several GB, and inputs allocated after them
        # streamed ~5% slower for the rest of the process.
        # Score kernel alone, cache rotated past the 256 MB Infinity Cache
        # (cold), and the same call on one input set that stays in that cache
        # (warm).
        sb = score_bytes(w)
        s_mean, s_med, s_p10, s_p90, s_b2b = time_score_rotating(qj, torch, w, sk, n_sets=4,
                                                                 iters=100)
        _, sw_med, _, _, _ = time_score_rotating(qj, torch, w, sk, n_sets=1, iters=100)
        del K
        torch.cuda.empty_cache()
        wl2 = wl.LONG_CTX
        sk2 = qj.make_sketch(wl2.seed, wl2.d, wl2.m, wl2.variant)
        sb2 = score_bytes(wl2)
        s2_mean, s2_med, s2_p10, s2_p90, s2_b2b = time_score_rotating(qj, torch, wl2, sk2,
                                                                      n_sets=2, iters=100)
        # decode-step attention on the scores (fused: the scores never reach HBM)
        att = {}
        for name, wa, sk_a, n_sets in (("attention_decode7b", w, sk, 2),
                                       ("attention_long_context", wl2, sk2, 2)):
            att[name] = (wa, attention_bytes(wa), n_sets,
                         time_attention_rotating(qj, torch, wa, sk_a, n_sets, iters=100))
        sk2.close()
        # the probes: torch's device copy and the plain-read ceilings
        copy_gbps = copy_peak_gbps(torch)
        result["copy_peak_GBps"] = copy_gbps
        result["roofline"]["frac_copy_peak"] = achieved / copy_gbps
        rc84 = read_ceiling(torch, int(sb), n_sets=4)
        rc302 = read_ceiling(torch, int(sb2), n_sets=2)
        rc612 = read_ceiling(torch, int(qbytes), n_sets=2)
        rc1359 = read_ceiling(torch, int(attention_bytes(wl2)), n_sets=2)
        result["read_ceiling"] = {"score_decode7b_bytes": rc84, "score_long_context_bytes": rc302,
                                  "quantize_bytes": rc612,
                                  "attention_long_context_bytes": rc1359}
        # the same byte counts split as the kernels split them into reads and
        # writes (the writes after the reads, as the score kernel defers them)
        sw1, sw2 = score_write_bytes(w), score_write_bytes(wl2)
        qw = quantize_write_bytes(w)
        rw84 = read_write_ceiling(torch, int(sb - sw1), int(sw1), n_sets=4)
        rw302 = read_write_ceiling(torch, int(sb2 - sw2), int(sw2), n_sets=2)
        rw612 = read_write_ceiling(torch, int(qbytes - qw), int(qw), n_sets=2)
        result["read_write_ceiling"] = {"score_decode7b_bytes": rw84,
                                        "score_long_context_bytes": rw302,
                                        "quantize_bytes": rw612}
        # the 7B attention moves the quantize's byte count within 0.1%
        att_rc = {"attention_decode7b": rc612, "attention_long_context": rc1359}
        if rc612:
            result["roofline"]["frac_read_ceiling"] = achieved / rc612["GBps"]
        if rw612:
            result["roofline"]["frac_read_write_ceiling"] = achieved / rw612["GBps"]
        result["score_decode7b"] = {"GBps": sb / s_med / 1e9, "frac_hbm": sb / s_med / 1e9 / HBM_PEAK_GBPS,
                                    "frac_read_ceiling": (sb / s_med / 1e9 / rc84["GBps"]
                                                          if rc84 else None),
                                    "frac_read_write_ceiling": (sb / s_med / 1e9 / rw84["GBps"]
                                                                if rw84 else None),
                                    "frac_copy_peak": sb / s_med / 1e9 / copy_gbps,
                                    "scores_per_s": w.groups * w.n_q * w.n_k / s_med,
                                    "mean_s": s_mean, "median_s": s_med, "p10_s": s_p10,
                                    "p90_s": s_p90, "bytes": sb,
                                    "rotation": "4 sets x 75.8 MB",
                                    "statistic": "median of 100 per-call HIP-event times",
                                    "back_to_back_mean_s": s_b2b,
                                    "warm_median_s": sw_med, "warm_GBps": sb / sw_med / 1e9}
        result["score_long_context"] = {"workload": wl2.name, "GBps": sb2 / s2_med / 1e9,
                                        "frac_hbm": sb2 / s2_med / 1e9 / HBM_PEAK_GBPS,
                                        "frac_read_ceiling": (sb2 / s2_med / 1e9 / rc302["GBps"]
                                                              if rc302 else None),
                                        "frac_read_write_ceiling": (
                                            sb2 / s2_med / 1e9 / rw302["GBps"] if rw302 else None),
                                        "frac_copy_peak": sb2 / s2_med / 1e9 / copy_gbps,
                                        "scores_per_s": wl2.groups * wl2.n_k / s2_med,
                                        "mean_s": s2_mean, "median_s": s2_med,
                                        "p10_s": s2_p10, "p90_s": s2_p90, "bytes": sb2,
                                        "rotation": "2 sets x 302 MB",
                                        "statistic": "median of 100 per-call HIP-event times",
                                        "back_to_back_mean_s": s2_b2b}
        for name, (wa, ab, n_sets, (a_mean, a_med, a_p10, a_p90)) in att.items():
            result[name] = {"workload": wa.name, "values": "bf16, d_v 128",
                            "GBps": ab / a_med / 1e9,
                            "frac_hbm": ab / a_med / 1e9 / HBM_PEAK_GBPS,
                            "frac_read_ceiling": (ab / a_med / 1e9 / att_rc[name]["GBps"]
                                                  if att_rc[name] else None),
                            "frac_copy_peak": ab / a_med / 1e9 / copy_gbps,
                            "keys_per_s": wa.groups * wa.n_k / a_med,
                            "mean_s": a_mean, "median_s": a_med, "p10_s": a_p10,
                            "p90_s": a_p90, "bytes": ab,
                            "timing": "HIP events around each call (partials + combine), "
                                      f"{n_sets} input sets rotated; rates from the median"}
        # the other quantize configurations (same 2,097,152-key cache size)
        for name, wq in (("quantize_prefill", wl.PREFILL), ("quantize_fqjl", wl.FQJL_7B),
                         ("quantize_fqjl_dither", wl.FQJL_7B_DITHER),
                         ("quantize_dfqjl", wl.DFQJL_7B), ("quantize_pfqjl", wl.PFQJL_7B)):
            tq, bq = time_quantize(qj, torch, wq)
            result[name] = {"workload": wq.name, "sketch": wq.variant, "rho": wq.rho,
                            "mean_s": tq, "keys_per_s": wq.n_keys / tq, "GBps": bq / tq / 1e9,
                            "frac_hbm": bq / tq / 1e9 / HBM_PEAK_GBPS,
                            "frac_copy_peak": bq / tq / 1e9 / copy_gbps,
                            "bound": "hbm" if wq.variant == "dense" else "alu",
                            "timing": "10 launches back to back"}
        result["decode_time"] = decode_time_extras(qj, torch, w, sk)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, K_host, args.cpu_seconds)
    sk.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
