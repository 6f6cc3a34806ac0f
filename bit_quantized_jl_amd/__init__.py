"""bit_quantized_jl_amd: the QJL key-cache sketch on AMD MI355X (gfx950).

A thin Python layer over libqjl (include/qjl.h): quantize keys to packed sign
bits plus norms, project queries, estimate attention scores and form the
decode-step attention output on them, all in hand-written HIP kernels.
"""
from ._lib import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_F32,
    ERR_DEVICE,
    ERR_INVALID_ARGUMENT,
    ERR_OUT_OF_MEMORY,
    ERR_UNSUPPORTED,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    OK,
    QJLError,
    Sketch,
    decode_attention,
    decode_attention_noalloc,
    decode_attention_workspace_size,
    destroy_sketch,
    generate_sketch_host,
    load,
    make_sketch,
    project_query,
    quantize_keys,
    quantize_keys_into,
    score,
    sketch_export,
    status_string,
    version,
)
