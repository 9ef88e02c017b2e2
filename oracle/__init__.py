"""fp64 CPU oracle for weight-absorbed MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers or constants) and imports
nothing from ``decode_attention_absorbed_amd``.

Every function here is pinned by the ``-m "not gpu"`` tests against
something other than itself (brute force, closed forms, the unabsorbed
multi-head form, scipy's softmax, invariants); none is "parity unpinned".
The FP8 variant (``mla_oracle_fp8``) is pinned against the OCP E4M3/E8M0
definitions, torch's float8_e4m3fn conversion and the bf16 reference on
inputs whose quantization is exact (tests/test_oracle_fp8.py).
"""
from .mla_oracle import (  # noqa: F401
    absorb_query,
    attend_rows,
    brute_force_ref,
    gather_kv_rows,
    lse_combine_ref,
    mha_unabsorbed_ref,
    mla_decode_ref,
    mla_decode_split_ref,
    visible_keys,
)
from .mla_oracle_fp8 import (  # noqa: F401
    E4M3_MAX,
    E4M3_REL_RMS,
    E4M3_REL_RMS_AVG,
    dequantize_cache,
    dequantize_query,
    e4m3_decode,
    e4m3_round,
    e4m3_table,
    e4m3_value,
    e8m0_decode,
    fp8_weight_error_rms,
    mla_decode_fp8_ref,
    query_exponent,
    quantize_query,
)
