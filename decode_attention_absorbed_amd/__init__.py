"""Weight-absorbed MLA decode attention for AMD Instinct MI355X (gfx950).

The computation lives in libmla_decode.so (hand-written HIP kernels and a C
ABI, declared in include/mla_decode.h); this package holds its sources, its
build step, a ctypes binding with the same function names, and the
FLOP/byte accounting used for roofline reporting.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    MLAError,
    Plan,
    lib,
    mla_decode,
    mla_decode_noalloc,
    mla_decode_variant,
    MLA_RESCALE_LAZY,
    MLA_RESCALE_POW2,
    mla_decode_plan,
    mla_decode_plan_host,
    mla_decode_workspace_bytes,
    mla_prolog,
    mla_o_project,
    mla_o_project_workspace_bytes,
    mla_up_project,
)
