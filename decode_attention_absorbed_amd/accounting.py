"""Algorithmic FLOP and byte counts of absorbed-MLA decode, and MI355X peaks.

FLOPs follow the convention of the Huawei Ascend report's MLA time model
(section 7.2): each (query, head, key) pair costs 2 x 576 multiply-adds for
QK^T and 2 x 512 for PV, i.e. 2 * (576 + 512) FLOPs.  The report counts every
query against all L keys; by default this module counts only the keys a query
may see (query j of a request with L keys sees L - q_len + 1 + j).

Bytes are the compulsory HBM traffic: the cached rows of every request
(576 bf16 each, or 576 E4M3 codes plus one scale byte for the FP8 cache), the
queries, the fp32 outputs and lse, the block table entries read and the
sequence lengths.  Partials and re-reads are not counted, so they show up as
a lower roofline fraction.
"""
from __future__ import annotations

from typing import Sequence

D_QK, D_V = 576, 512
ROW_BYTES = D_QK * 2  # bf16 row per cached token
ROW_BYTES_FP8 = D_QK + 1  # E4M3 codes + the E8M0 scale byte

# MI355X published peaks (dense): HBM3E 8 TB/s, bf16 MFMA 2.5 PFLOP/s, fp8 MFMA 5.0 PFLOP/s.
PEAK_HBM_BYTES_PER_S = 8.0e12
PEAK_BF16_FLOPS = 2.5e15
PEAK_FP8_FLOPS = 5.0e15


def visible_key_count(seq_lens: Sequence[int], q_len: int) -> int:
    return sum(q_len * (int(L) - q_len + 1) + q_len * (q_len - 1) // 2 for L in seq_lens)


def flops(seq_lens: Sequence[int], heads: int, q_len: int, visible: bool = True) -> int:
    keys = visible_key_count(seq_lens, q_len) if visible else q_len * sum(int(L) for L in seq_lens)
    return 2 * (D_QK + D_V) * heads * keys


def kv_bytes(seq_lens: Sequence[int], kv: str = "bf16") -> int:
    return (ROW_BYTES_FP8 if kv == "fp8" else ROW_BYTES) * sum(int(L) for L in seq_lens)


def algorithmic_bytes(seq_lens: Sequence[int], heads: int, q_len: int, page: int, kv: str = "bf16") -> int:
    B = len(seq_lens)
    rows = B * q_len * heads
    q = rows * D_QK * 2
    out = rows * D_V * 4 + rows * 4
    bt = 4 * sum(-(-int(L) // page) for L in seq_lens) + 4 * B
    return kv_bytes(seq_lens, kv) + q + out + bt


def roofline_seconds(seq_lens: Sequence[int], heads: int, q_len: int, page: int, kv: str = "bf16") -> dict:
    """Time at the HBM and MFMA peaks (bf16 or fp8 matrix rate) and which one binds."""
    f = flops(seq_lens, heads, q_len)
    b = algorithmic_bytes(seq_lens, heads, q_len, page, kv)
    t_hbm = b / PEAK_HBM_BYTES_PER_S
    t_mfma = f / (PEAK_FP8_FLOPS if kv == "fp8" else PEAK_BF16_FLOPS)
    return {
        "flops": f,
        "bytes": b,
        "t_hbm": t_hbm,
        "t_mfma": t_mfma,
        "bound": "hbm" if t_hbm >= t_mfma else "mfma",
        "t_bound": max(t_hbm, t_mfma),
    }


# ---- the steps next to the decode: compulsory bytes (each is bound by HBM) ------------------

D_NOPE, D_ROPE = 128, 64  # per-head query part before the absorption, and the RoPE part


def prolog_bytes(rows: int, heads: int, kv: str = "bf16") -> int:
    """Absorbed-query projection + RoPE + cache append for `rows` = B * q_len
    new tokens: W_UK (H x 128 x 512 bf16), q_nope in (128 bf16) and the
    absorbed query out (512 bf16) per row and head, q_pe in and out (64 bf16
    each), c_kv (512 bf16) and k_pe (64 bf16) in and the cache row out per
    token, the norm weight and one RoPE table row (64 fp32) per token."""
    w = heads * D_NOPE * D_V * 2
    per_head = rows * heads * (D_NOPE * 2 + D_V * 2 + 2 * D_ROPE * 2)
    row_out = ROW_BYTES_FP8 if kv == "fp8" else ROW_BYTES
    per_token = rows * ((D_V + D_ROPE) * 2 + row_out + 64 * 4 + 4 + 4)
    return w + per_head + per_token + D_V * 2


def up_project_bytes(rows: int, heads: int) -> int:
    """Value up-projection: W_UV (H x 128 x 512 bf16), the fp32 attention output
    in (512 per row and head) and the bf16 result out (128)."""
    return heads * D_NOPE * D_V * 2 + rows * heads * (D_V * 4 + D_NOPE * 2)


HIDDEN = 7168  # DeepSeek-V3's model width: the output projection's rows


def o_project_bytes(rows: int, heads: int, hidden: int = HIDDEN) -> int:
    """Output projection: W_O (hidden x H*128 bf16), its bf16 input (H*128 per
    row) and bf16 output (hidden per row); the fp32 partial sums over slices
    of the input width are not compulsory and are not counted."""
    k = heads * D_NOPE
    return hidden * k * 2 + rows * (k + hidden) * 2
