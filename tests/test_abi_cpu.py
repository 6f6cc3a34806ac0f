"""The C ABI on the CPU: the library loads, exports every declared symbol,
validates arguments before touching a GPU, and its host sketch generator
matches the oracle's independent one bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_jl_amd as qj
from bit_quantized_jl_amd import _lib
from oracle import sketch as osk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qjl.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(qjl_[a-z0-9_]+)\s*\(", txt)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = qj.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    # and the shared object's dynamic symbol table lists them (extern "C")
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qj.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (qjl_[a-z0-9_]+)$", out, flags=re.M))
    assert set(names) <= exported


def test_status_strings_and_version():
    for code, name in [(0, "QJL_OK"), (1, "QJL_ERR_INVALID_ARGUMENT"), (2, "QJL_ERR_UNSUPPORTED"),
                       (3, "QJL_ERR_OUT_OF_MEMORY"), (4, "QJL_ERR_DEVICE")]:
        assert qj.status_string(code) == name
    assert qj.status_string(99) == "QJL_ERR_UNKNOWN"
    assert "gfx950" in qj.version()


@pytest.mark.parametrize("args,expect", [
    ((0, 128, 250, 0, 0.0), 1),      # m % 32 != 0
    ((0, 128, 0, 0, 0.0), 1),        # m = 0
    ((0, 0, 256, 0, 0.0), 1),        # d = 0
    ((0, 128, 256, 7, 0.0), 1),      # bad variant
    ((0, 128, 256, 0, -0.1), 1),     # rho < 0
    ((0, 128, 256, 0, float("nan")), 1),
    ((0, 128, 256, 0, float("inf")), 1),
    ((0, 1024, 256, 0, 0.0), 2),     # dense d too large
    ((0, 128, 16384, 0, 0.0), 2),    # m too large
    ((0, 96, 192, 1, 0.0), 2),       # FQJL d not a power of two
    ((0, 128, 320, 1, 0.0), 2),      # FQJL m % d != 0
    ((0, 4, 32, 1, 0.0), 2),         # FQJL d < 8
    ((0, 512, 1024, 1, 0.0), 2),     # FQJL d > 256
    ((0, 256, 384, 1, 0.0), 2),      # FQJL m % d != 0 at d = 256
    ((0, 128, 256, 4, 0.0), 1),      # no variant 4
    ((0, 128, 256, 2, 0.0), 1),      # D-FQJL needs dither
    ((0, 128, 256, 3, 0.1), 1),      # P-FQJL has none
    ((0, 96, 192, 2, 0.1), 2),       # D-FQJL d not a power of two
])
def test_make_sketch_validation(args, expect):
    lib = qj.load()
    out = ctypes.c_void_p(123)
    st = lib.qjl_make_sketch(*args, ctypes.byref(out))
    assert st == expect
    assert out.value is None


def test_make_sketch_null_out_and_no_gpu():
    lib = qj.load()
    assert lib.qjl_make_sketch(0, 128, 256, 0, 0.0, None) == 1
    import torch
    if not torch.cuda.is_available():
        out = ctypes.c_void_p()
        assert lib.qjl_make_sketch(0, 128, 256, 0, 0.0, ctypes.byref(out)) == qj.ERR_DEVICE
        assert out.value is None


def test_null_handles_rejected():
    lib = qj.load()
    assert lib.qjl_destroy_sketch(None) == 1
    assert lib.qjl_sketch_info(None, None, None, None, None, None, None) == 1
    assert lib.qjl_sketch_export(None, None, None) == 1
    assert lib.qjl_quantize_keys(None, None, 1, 4, 0, None, None, None) == 1
    assert lib.qjl_quantize_keys_into(None, None, 1, 2, 1, 8, 7, 0, None, None, None) == 1
    assert lib.qjl_project_query(None, None, 1, 4, None, None) == 1
    assert lib.qjl_score(None, None, None, None, 1, 1, 1, None, None) == 1
    sz = ctypes.c_size_t(7)
    assert lib.qjl_decode_attention_workspace_size(None, 1, 1, 1, 128, ctypes.byref(sz)) == 1
    assert lib.qjl_decode_attention(None, None, None, None, None, 1, 128, 1, 1, 1, 1.0, None, 0,
                                    None, None) == 1


@pytest.mark.parametrize("seed,d,m", [(0, 128, 256), (0, 128, 512), (7, 16, 32), (3, 100, 64)])
def test_host_dense_sketch_equals_oracle(seed, d, m):
    got = qj.generate_sketch_host(seed, d, m, "dense")
    ref = osk.make_dense(seed, d, m, rho=0.1)
    assert np.array_equal(got["S_f32"].astype(np.float64), ref.S32)
    assert np.array_equal(got["S_bf16"], osk.bf16_bits(ref.S16))
    assert np.array_equal(got["dither_mag"].astype(np.float64), ref.dmag)


@pytest.mark.parametrize("variant", ["fqjl", "dfqjl", "pfqjl"])
@pytest.mark.parametrize("seed,d,m", [(0, 128, 256), (5, 8, 32), (9, 64, 192), (2, 128, 512),
                                      (4, 256, 512)])
def test_host_fqjl_params_equal_oracle(seed, d, m, variant):
    got = qj.generate_sketch_host(seed, d, m, variant)
    ref = osk.make_sketch(seed, d, m, variant, 0.0 if variant == "pfqjl" else 0.1)
    assert np.array_equal(got["D"].astype(np.float64), ref.D)
    assert np.array_equal(got["P"].astype(np.int64), ref.P)
    assert np.array_equal(got["G"].astype(np.float64), ref.G)
    if ref.dmag is not None:
        assert np.array_equal(got["dither_mag"].astype(np.float64), ref.dmag)


def test_host_generation_validates():
    with pytest.raises(qj.QJLError) as e:
        qj.generate_sketch_host(0, 128, 100, "dense")
    assert e.value.status == qj.ERR_INVALID_ARGUMENT
    with pytest.raises(qj.QJLError) as e:
        qj.generate_sketch_host(0, 96, 192, "fqjl")
    assert e.value.status == qj.ERR_UNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises((ValueError, RuntimeError, qj.QJLError)):
        sk = _lib.Sketch(0, 0, 128, 256, "dense", 0.0)
        qj.quantize_keys(sk, torch.zeros(4, 128))


class _DevStub:
    """Stands in for a contiguous GPU tensor (shape and dtype only): the
    binding's checks run on it without a GPU, and reaching a launch (which
    reads data_ptr) fails the test."""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)

    def numel(self):
        return int(np.prod(self.shape))

    def data_ptr(self):
        raise AssertionError("a launch was reached with a mistyped buffer")


@pytest.mark.parametrize("bad", ["float16", "bfloat16", "int16", "float64", "uint8"])
def test_binding_rejects_mistyped_buffers_before_launch(bad):
    # A narrower dtype with enough elements would let the kernels write 4-byte
    # words past the allocation; a wider one would be misread.  Every buffer
    # the library reads or writes is checked before the call.
    import types

    import torch
    bad = getattr(torch, bad)
    n, d, m = 64, 128, 256
    sk = types.SimpleNamespace(d=d, m=m, handle=None)
    K = _DevStub((n, d), torch.bfloat16)
    f32 = lambda *s: _DevStub(s, torch.float32)
    words = lambda *s: _DevStub(s, torch.int32)
    wrong = lambda *s: _DevStub((2 * int(np.prod(s)),), bad)   # twice the elements
    calls = [
        lambda: qj.quantize_keys(sk, K, norms_out=wrong(n), bits_out=words(n, m // 32)),
        lambda: qj.quantize_keys(sk, K, norms_out=f32(n), bits_out=wrong(n, m // 32)),
        lambda: qj.quantize_keys_into(sk, K, 1, wrong(n), words(n, m // 32), n, 0),
        lambda: qj.quantize_keys_into(sk, K, 1, f32(n), wrong(n, m // 32), n, 0),
        lambda: qj.project_query(sk, K, Sq_out=wrong(n, m)),
        lambda: qj.score(sk, f32(1, m), words(n, m // 32), f32(n), 1, 1, n,
                         scores_out=wrong(1, 1, n)),
        lambda: qj.score(sk, wrong(1, m), words(n, m // 32), f32(n), 1, 1, n,
                         scores_out=f32(1, 1, n)),
        lambda: qj.score(sk, f32(1, m), wrong(n, m // 32), f32(n), 1, 1, n,
                         scores_out=f32(1, 1, n)),
        lambda: qj.score(sk, f32(1, m), words(n, m // 32), wrong(n), 1, 1, n,
                         scores_out=f32(1, 1, n)),
    ]
    for call in calls:
        with pytest.raises(TypeError):
            call()


def test_binding_rejects_short_buffers_before_launch():
    import types

    import torch
    n, d, m = 64, 128, 256
    sk = types.SimpleNamespace(d=d, m=m, handle=None)
    K = _DevStub((n, d), torch.bfloat16)
    with pytest.raises(ValueError):
        qj.quantize_keys(sk, K, norms_out=_DevStub((n - 1,), torch.float32),
                         bits_out=_DevStub((n, m // 32), torch.int32))
    with pytest.raises(ValueError):
        qj.score(sk, _DevStub((1, m), torch.float32), _DevStub((n, m // 32), torch.int32),
                 _DevStub((n,), torch.float32), 1, 1, n,
                 scores_out=_DevStub((n - 1,), torch.float32))


def test_probe_library_loads():
    # the benchmark's plain read kernels: a separate library, not part of libqjl
    from bit_quantized_jl_amd import build as b
    assert os.path.exists(b.PROBE_LIB)
    lib = ctypes.CDLL(b.PROBE_LIB)
    fn = lib.qjl_probe_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    # argument checks happen before any HIP call
    assert fn(None, 16, 0, 4, 1, None, None) == 1
    assert fn(16, 15, 0, 4, 1, 16, None) == 1          # bytes not a multiple of 16
    assert fn(16, 16, 2, 4, 1, 16, None) == 1          # bad pattern
    assert fn(16, 16, 0, 3, 1, 16, None) == 1          # bad unroll
    assert "qjl_probe_read" not in {n for n in dir(qj.load()) if n.startswith("qjl_")}
