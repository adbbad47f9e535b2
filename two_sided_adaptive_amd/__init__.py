"""GPTQ-2D two-sided adaptive rounding on AMD Instinct MI355X (gfx950).

The computation lives in libgptq2d.so (HIP kernels behind the C ABI of
include/gptq2d.h); this package only marshals torch device tensors into it.
"""
from ._binding import (  # noqa: F401
    F32,
    F64,
    GPTQ2DError,
    LIB_PATH,
    factor,
    gram_accumulate,
    gram_accumulate_batched,
    load_library,
    pack,
    packed_gemv,
    profile_enable,
    profile_read,
    profile_task_classes,
    quantize,
    quantize3,
    quantize_factored,
    quantize_noalloc,
    unpack,
    workspace_bytes,
)
