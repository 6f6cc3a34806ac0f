"""ctypes binding of libqjl (argument marshalling only).

Every function here has the name of a C entry point in include/qjl.h minus
the ``qjl_`` prefix.  Device buffers are torch tensors on the sketch's GPU;
torch supplies memory and the current stream, the library does all of the
computation.  Packed sign bits are stored in int32 tensors (the bit pattern
of the uint32 words of the C ABI).

The library must be built (``python -m bit_quantized_jl_amd.build``);
loading fails loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqjl.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_OUT_OF_MEMORY = 3
ERR_DEVICE = 4

VARIANTS = {"dense": 0, "fqjl": 1, "dfqjl": 2, "pfqjl": 3}
DTYPE_F32 = 0
DTYPE_BF16 = 1

_lib: Optional[ctypes.CDLL] = None


class QJLError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)}")


def _declare(lib: ctypes.CDLL) -> None:
    c = ctypes
    vp, i32, i64, u64, f32 = c.c_void_p, c.c_int32, c.c_int64, c.c_uint64, c.c_float
    sig = {
        "qjl_make_sketch": (c.c_int, [u64, i32, i32, i32, f32, c.POINTER(vp)]),
        "qjl_destroy_sketch": (c.c_int, [vp]),
        "qjl_sketch_info": (c.c_int, [vp, c.POINTER(u64), c.POINTER(i32), c.POINTER(i32),
                                      c.POINTER(i32), c.POINTER(f32), c.POINTER(i32)]),
        "qjl_sketch_export": (c.c_int, [vp, vp, vp]),
        "qjl_generate_sketch_host": (c.c_int, [u64, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "qjl_quantize_keys": (c.c_int, [vp, vp, i32, i64, i64, vp, vp, vp]),
        "qjl_quantize_keys_into": (c.c_int, [vp, vp, i32, i64, i64, i64, i64, i64, vp, vp, vp]),
        "qjl_project_query": (c.c_int, [vp, vp, i32, i64, vp, vp]),
        "qjl_score": (c.c_int, [vp, vp, vp, vp, i64, i64, i64, vp, vp]),
        "qjl_decode_attention_workspace_size": (c.c_int, [vp, i64, i64, i64, i32,
                                                          c.POINTER(c.c_size_t)]),
        "qjl_decode_attention": (c.c_int, [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64, f32,
                                           vp, c.c_size_t, vp, vp]),
        "qjl_decode_attention_noalloc": (c.c_int, [vp, vp, vp, vp, vp, i32, i32, i64, i64, i64,
                                                   f32, vp, vp]),
        "qjl_status_string": (c.c_char_p, [c.c_int]),
        "qjl_version": (c.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def load() -> ctypes.CDLL:
    """Load libqjl.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_jl_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(LIB_PATH)
        _declare(lib)
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().qjl_status_string(int(status)).decode()


def version() -> str:
    return load().qjl_version().decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise QJLError(status, what)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev_tensor(t, name: str, ndim: int | None = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return t


def _f32_types():
    import torch
    return (torch.float32,)


def _word_types():
    """Tensor dtypes that hold the uint32 sign words (4-byte integers)."""
    import torch
    return tuple(t for t in (torch.int32, getattr(torch, "uint32", None)) if t is not None)


def _buffer(t, name: str, dtypes: tuple, numel: int):
    """A device buffer the library reads or writes `numel` 4-byte elements of:
    contiguous, on the GPU, of one of `dtypes` and at least that large.  The
    kernels write whole 4-byte words, so a narrower dtype with enough elements
    would be overrun; it is rejected here, before any launch."""
    _dev_tensor(t, name)
    if t.dtype not in dtypes:
        names = " or ".join(str(d) for d in dtypes)
        raise TypeError(f"{name} must be {names}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    return t


class Sketch:
    """An owned qjl_sketch handle (see qjl_make_sketch)."""

    def __init__(self, handle: int, seed: int, d: int, m: int, variant: str, rho: float):
        self._h = ctypes.c_void_p(handle)
        self.seed, self.d, self.m, self.variant, self.rho = seed, d, m, variant, rho

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ValueError("sketch already destroyed")
        return self._h

    def info(self) -> dict:
        seed, d, m, var, dev = (ctypes.c_uint64(), ctypes.c_int32(), ctypes.c_int32(),
                                ctypes.c_int32(), ctypes.c_int32())
        rho = ctypes.c_float()
        _check(load().qjl_sketch_info(self.handle, ctypes.byref(seed), ctypes.byref(d),
                                      ctypes.byref(m), ctypes.byref(var), ctypes.byref(rho),
                                      ctypes.byref(dev)), "qjl_sketch_info")
        return {"seed": seed.value, "d": d.value, "m": m.value, "variant": var.value,
                "rho": rho.value, "device": dev.value}

    def close(self) -> None:
        if self._h:
            h, self._h = self._h, ctypes.c_void_p(0)
            _check(load().qjl_destroy_sketch(h), "qjl_destroy_sketch")

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                load().qjl_destroy_sketch(self._h)
                self._h = ctypes.c_void_p(0)
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def make_sketch(seed: int, d: int, m: int, variant: str = "dense", rho: float = 0.0) -> Sketch:
    h = ctypes.c_void_p()
    _check(load().qjl_make_sketch(int(seed), int(d), int(m), VARIANTS[variant], float(rho),
                                  ctypes.byref(h)), "qjl_make_sketch")
    return Sketch(h.value, seed, d, m, variant, rho)


def destroy_sketch(sk: Sketch) -> None:
    sk.close()


def sketch_export(sk: Sketch, bf16: bool = False):
    """(S_f32 [m, d] float32, S_bf16 [m, d] uint16 or None) on the host."""
    s32 = np.empty((sk.m, sk.d), dtype=np.float32)
    s16 = np.empty((sk.m, sk.d), dtype=np.uint16) if bf16 else None
    _check(load().qjl_sketch_export(sk.handle, s32.ctypes.data,
                                    None if s16 is None else s16.ctypes.data),
           "qjl_sketch_export")
    return s32, s16


def generate_sketch_host(seed: int, d: int, m: int, variant: str = "dense") -> dict:
    """Host-only draw of the sketch parameters (works without a GPU)."""
    out = {}
    dmag = np.empty(max(m, 0), np.float32)
    if variant == "dense":
        s32 = np.empty((m, d), np.float32)
        s16 = np.empty((m, d), np.uint16)
        _check(load().qjl_generate_sketch_host(seed, d, m, 0, s32.ctypes.data, s16.ctypes.data,
                                               None, None, None, dmag.ctypes.data),
               "qjl_generate_sketch_host")
        out.update(S_f32=s32, S_bf16=s16, dither_mag=dmag)
    else:
        nb = m // d if d > 0 else 0
        D = np.empty((nb, d), np.int8)
        P = np.empty((nb, d), np.int32)
        G = np.empty((nb, d), np.float32)
        _check(load().qjl_generate_sketch_host(seed, d, m, VARIANTS[variant], None, None,
                                               D.ctypes.data, P.ctypes.data, G.ctypes.data,
                                               dmag.ctypes.data),
               "qjl_generate_sketch_host")
        out.update(D=D, P=P, G=G, dither_mag=dmag)
    return out


def quantize_keys(sk: Sketch, K, key_index_base: int = 0, norms_out=None, bits_out=None,
                  stream=None):
    """Quantize keys K [n, d] (float32 or bfloat16) -> (norms [n] float32,
    bits [n, m/32] int32 holding the uint32 sign words)."""
    import torch
    _dev_tensor(K, "K", 2)
    n = K.shape[0]
    if K.shape[1] != sk.d:
        raise ValueError(f"K has {K.shape[1]} columns, sketch d = {sk.d}")
    if norms_out is None:
        norms_out = torch.empty(n, dtype=torch.float32, device=K.device)
    if bits_out is None:
        bits_out = torch.empty((n, sk.m // 32), dtype=torch.int32, device=K.device)
    _buffer(norms_out, "norms_out", _f32_types(), n)
    _buffer(bits_out, "bits_out", _word_types(), n * (sk.m // 32))
    _check(load().qjl_quantize_keys(sk.handle, _ptr(K), _dtype_code(K), n, int(key_index_base),
                                    _ptr(norms_out), _ptr(bits_out), _stream(stream)),
           "qjl_quantize_keys")
    return norms_out, bits_out


def quantize_keys_into(sk: Sketch, K, n_groups: int, norms_cache, bits_cache,
                       cache_rows_per_group: int, first_row: int, key_index_base: int = 0,
                       stream=None):
    """Quantize K [n_groups * keys_per_group, d] into a key cache laid out by
    group: key i of group g goes to row g * cache_rows_per_group + first_row + i
    of norms_cache [n_groups * cache_rows_per_group] (float32) and bits_cache
    [n_groups * cache_rows_per_group, m/32] (int32 words).  Returns the cache."""
    _dev_tensor(K, "K", 2)
    if K.shape[1] != sk.d:
        raise ValueError(f"K has {K.shape[1]} columns, sketch d = {sk.d}")
    if n_groups <= 0 or K.shape[0] % n_groups != 0:
        raise ValueError("K's rows must split evenly into n_groups groups")
    kpg = K.shape[0] // n_groups
    rows = n_groups * int(cache_rows_per_group)
    _buffer(norms_cache, "norms_cache", _f32_types(), rows)
    _buffer(bits_cache, "bits_cache", _word_types(), rows * (sk.m // 32))
    _check(load().qjl_quantize_keys_into(sk.handle, _ptr(K), _dtype_code(K), int(n_groups), kpg,
                                         int(cache_rows_per_group), int(first_row),
                                         int(key_index_base), _ptr(norms_cache),
                                         _ptr(bits_cache), _stream(stream)),
           "qjl_quantize_keys_into")
    return norms_cache, bits_cache


def project_query(sk: Sketch, q, Sq_out=None, stream=None):
    """Project queries q [n, d] -> Sq [n, m] float32 (not quantized)."""
    import torch
    _dev_tensor(q, "q", 2)
    n = q.shape[0]
    if q.shape[1] != sk.d:
        raise ValueError(f"q has {q.shape[1]} columns, sketch d = {sk.d}")
    if Sq_out is None:
        Sq_out = torch.empty((n, sk.m), dtype=torch.float32, device=q.device)
    _buffer(Sq_out, "Sq_out", _f32_types(), n * sk.m)
    _check(load().qjl_project_query(sk.handle, _ptr(q), _dtype_code(q), n, _ptr(Sq_out),
                                    _stream(stream)), "qjl_project_query")
    return Sq_out


def score(sk: Sketch, Sq, bits, norms, n_groups: int, n_q: int, n_k: int, scores_out=None,
          stream=None):
    """Estimated scores [n_groups, n_q, n_k] float32."""
    import torch
    _buffer(Sq, "Sq", _f32_types(), n_groups * n_q * sk.m)
    _buffer(bits, "bits", _word_types(), n_groups * n_k * (sk.m // 32))
    _buffer(norms, "norms", _f32_types(), n_groups * n_k)
    if scores_out is None:
        scores_out = torch.empty((n_groups, n_q, n_k), dtype=torch.float32, device=Sq.device)
    _buffer(scores_out, "scores_out", _f32_types(), n_groups * n_q * n_k)
    _check(load().qjl_score(sk.handle, _ptr(Sq), _ptr(bits), _ptr(norms), int(n_groups),
                            int(n_q), int(n_k), _ptr(scores_out), _stream(stream)),
           "qjl_score")
    return scores_out


def decode_attention_workspace_size(sk: Sketch, n_groups: int, n_q: int, n_k: int,
                                    d_v: int) -> int:
    """Bytes of device workspace qjl_decode_attention needs for these counts."""
    out = ctypes.c_size_t(0)
    _check(load().qjl_decode_attention_workspace_size(sk.handle, int(n_groups), int(n_q),
                                                      int(n_k), int(d_v), ctypes.byref(out)),
           "qjl_decode_attention_workspace_size")
    return int(out.value)


def decode_attention(sk: Sketch, Sq, bits, norms, V, n_groups: int, n_q: int, n_k: int,
                     softmax_scale: float, workspace=None, out=None, stream=None):
    """Attention outputs [n_groups, n_q, d_v] float32 from the QJL scores.

    V is [n_groups, n_k, d_v] float32 or bfloat16.  The workspace (a uint8
    GPU tensor) is allocated here when not given.
    """
    import torch
    _dev_tensor(V, "V")
    if V.dim() < 1:
        raise ValueError("V must have a last dimension d_v")
    d_v = int(V.shape[-1])
    _buffer(Sq, "Sq", _f32_types(), n_groups * n_q * sk.m)
    _buffer(bits, "bits", _word_types(), n_groups * n_k * (sk.m // 32))
    _buffer(norms, "norms", _f32_types(), n_groups * n_k)
    _buffer(V, "V", (torch.float32, torch.bfloat16), n_groups * n_k * d_v)
    need = decode_attention_workspace_size(sk, n_groups, n_q, n_k, d_v)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Sq.device)
    _dev_tensor(workspace, "workspace")
    if out is None:
        out = torch.empty((n_groups, n_q, d_v), dtype=torch.float32, device=Sq.device)
    _buffer(out, "out", _f32_types(), n_groups * n_q * d_v)
    nbytes = workspace.numel() * workspace.element_size()
    _check(load().qjl_decode_attention(sk.handle, _ptr(Sq), _ptr(bits), _ptr(norms), _ptr(V),
                                       _dtype_code(V), d_v, int(n_groups), int(n_q), int(n_k),
                                       float(softmax_scale), _ptr(workspace), nbytes,
                                       _ptr(out), _stream(stream)),
           "qjl_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # QJL_NOALLOC_SCRATCH_BYTES


def decode_attention_noalloc(sk: Sketch, Sq, bits, norms, V, n_groups: int, n_q: int, n_k: int,
                             softmax_scale: float, out, stream=None):
    """decode_attention with the library's per-GPU scratch as its workspace:
    no allocation anywhere in the call (the caller passes `out`, float32
    [n_groups, n_q, d_v]).  Calls that overlap on one GPU race on the scratch."""
    import torch
    _dev_tensor(V, "V")
    if V.dim() < 1:
        raise ValueError("V must have a last dimension d_v")
    d_v = int(V.shape[-1])
    _buffer(Sq, "Sq", _f32_types(), n_groups * n_q * sk.m)
    _buffer(bits, "bits", _word_types(), n_groups * n_k * (sk.m // 32))
    _buffer(norms, "norms", _f32_types(), n_groups * n_k)
    _buffer(V, "V", (torch.float32, torch.bfloat16), n_groups * n_k * d_v)
    _buffer(out, "out", _f32_types(), n_groups * n_q * d_v)
    _check(load().qjl_decode_attention_noalloc(sk.handle, _ptr(Sq), _ptr(bits), _ptr(norms),
                                               _ptr(V), _dtype_code(V), d_v, int(n_groups),
                                               int(n_q), int(n_k), float(softmax_scale),
                                               _ptr(out), _stream(stream)),
           "qjl_decode_attention_noalloc")
    return out
