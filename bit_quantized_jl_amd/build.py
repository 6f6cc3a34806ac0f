"""Build libqjl.so (HIP for gfx950) in-tree with hipcc.

    python -m bit_quantized_jl_amd.build

Each source is compiled to an object in parallel, then linked into
bit_quantized_jl_amd/libqjl.so.  All HIP code is built with packed fp32
instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqjl.so")
PROBE_LIB = os.path.join(HERE, "libqjl_probe.so")
ARCH = os.environ.get("QJL_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.relpath(src, CSRC).replace(os.sep, "_") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON, *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def probe_sources() -> list[str]:
    d = os.path.join(CSRC, "probe")
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """Build libqjl.so (the library) and libqjl_probe.so (the benchmark's
    plain read kernels, kept out of the library)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    psrcs = probe_sources()
    workers = min(len(srcs) + len(psrcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
