"""Plain fp64 reference for the steps around the decode attention (numpy).

TEST INFRASTRUCTURE ONLY: see the package docstring.

The Huawei report ("DeepSeek V3/R1 inference deployment best practices on
Ascend servers", section 6.1, the paragraph on the operators before MLA)
fuses what precedes the decode attention into one "MLAProlog" operator with
the weights absorbed, and the CloudMatrix384 digest (its MLA optimization
paragraph) lists the fused parts: RMSNorm, the Q/K/V projections and RoPE.
The same report's decode data flow ends MLA with the output projection
(section 3.2.1, the O Proj of its figures).  This module fixes the part of
that chain that sits next to the decode attention; the readings (listed with
the others in the design notes):

  * prolog, per decode step, from the already projected per-head query
    (q_nope 128 + q_pe 64 per head) and the new tokens' compressed KV
    (c_kv 512 before its RMSNorm, k_pe 64 before RoPE):
      q_nope_absorbed = W_UK^T q_nope per head (the absorption);
      q_pe  = RoPE(q_pe) at the token's position;
      row   = [RMSNorm(c_kv) * w | RoPE(k_pe)], rounded to bf16, written to
              the paged cache at the token's position (and, for the FP8
              cache, quantized per token: the row's E8M0 exponent is the
              smallest f with amax * 2^-f <= 448, its codes the nearest E4M3
              values of row * 2^-f);
    positions: query token j of a request of L tokens (the q_len new ones
    included) sits at L - q_len + j;
  * RoPE rotates the pairs (x[2i], x[2i+1]) of the 64 rope dims by the angle
    of pair i at that position; the angles come in as a cos/sin table (so
    plain RoPE and frequency-scaled variants are the caller's table);
    RMSNorm is x / sqrt(mean(x^2) + eps) * w;
  * epilog: the value up-projection o_h = W_UV[h] out_h (128 wide per head),
    the input of the output projection; then the output projection itself,
    y = W_O [o_0 | o_1 | ... | o_{H-1}] (heads concatenated in order, W_O of
    shape [hidden, H * 128] as a linear layer stores it).
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from .mla_oracle import D_LATENT, D_ROPE, absorb_query
from .mla_oracle_fp8 import E4M3_MAX, e4m3_round, query_exponent


def rope_ref(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (x[..., 2i], x[..., 2i+1]) by the angle with cosine cos[..., i]
    and sine sin[..., i] (x [..., 64], cos/sin [..., 32] broadcastable)."""
    x = np.asarray(x, np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def rmsnorm_ref(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def positions(seq_lens: Sequence[int], q_len: int) -> np.ndarray:
    """[B, q_len]: position of query token j of request b (L_b - q_len + j)."""
    L = np.asarray(seq_lens, np.int64)[:, None]
    return L - q_len + np.arange(q_len)[None, :]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (ties to even), as float64."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def prolog_ref(
    q_nope128: np.ndarray,
    q_pe_raw: np.ndarray,
    W_UK: np.ndarray,
    c_kv_raw: np.ndarray,
    kv_norm_w: np.ndarray,
    rms_eps: float,
    k_pe_raw: np.ndarray,
    rope_cos: np.ndarray,
    rope_sin: np.ndarray,
    seq_lens: Sequence[int],
) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The prolog in fp64.

    q_nope128 [B, q_len, H, 128], q_pe_raw [B, q_len, H, 64], W_UK [H, 128, 512],
    c_kv_raw [B, q_len, 512], kv_norm_w [512], k_pe_raw [B, q_len, 64],
    rope_cos / rope_sin [max_pos, 32].
    Returns q_nope_absorbed [B, q_len, H, 512], q_pe [B, q_len, H, 64] (fp64)
    and the new cache rows [B, q_len, 576] rounded to bf16 (as float64).
    """
    B, q_len = q_nope128.shape[:2]
    pos = positions(seq_lens, q_len)
    cos, sin = np.asarray(rope_cos)[pos], np.asarray(rope_sin)[pos]  # [B, q_len, 32]
    q_abs = absorb_query(np.asarray(q_nope128, np.float64), np.asarray(W_UK, np.float64))
    q_pe = rope_ref(q_pe_raw, cos[:, :, None, :], sin[:, :, None, :])
    rows = np.concatenate([rmsnorm_ref(c_kv_raw, kv_norm_w, rms_eps), rope_ref(k_pe_raw, cos, sin)], axis=-1)
    return q_abs, q_pe, bf16_round(rows)


def append_ref(cache: np.ndarray, block_table: np.ndarray, seq_lens: Sequence[int], rows: np.ndarray) -> np.ndarray:
    """A copy of cache [num_pages, P, ...] with rows [B, q_len, ...] written at the
    new tokens' positions (token t of request b: slot t % P of page block_table[b, t // P])."""
    out = np.array(cache, copy=True)
    P = cache.shape[1]
    B, q_len = rows.shape[:2]
    pos = positions(seq_lens, q_len)
    for b in range(B):
        for j in range(q_len):
            t = int(pos[b, j])
            out[int(block_table[b, t // P]), t % P] = rows[b, j]
    return out


def quantize_row_fp8(row: np.ndarray) -> Tuple[np.ndarray, int]:
    """One cache row to (E4M3 codes [576], E8M0 scale byte): f = smallest integer
    with amax * 2^-f <= 448 (limited to [-127, 127]; f = 0 for a zero row)."""
    row = np.asarray(row, np.float64)
    f = min(max(query_exponent(np.abs(row).max()), -127), 127)
    return e4m3_round(np.clip(np.ldexp(row, -f), -E4M3_MAX, E4M3_MAX)), 127 + f


def up_project_ref(out: np.ndarray, W_UV: np.ndarray) -> np.ndarray:
    """o[..., h, :] = W_UV[h] @ out[..., h, :] (out [..., H, 512], W_UV [H, 128, 512])."""
    return np.einsum("...hc,hdc->...hd", np.asarray(out, np.float64), np.asarray(W_UV, np.float64))


def rope_table(theta: float, max_pos: int) -> Tuple[np.ndarray, np.ndarray]:
    """Plain RoPE angles: pair i of position p turns by p * theta^(-2i/64)."""
    inv = theta ** (-np.arange(0, D_ROPE, 2, dtype=np.float64) / D_ROPE)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def o_project_ref(o: np.ndarray, W_O: np.ndarray) -> np.ndarray:
    """y[..., :] = W_O @ concat_h o[..., h, :] (o [..., H, 128], W_O [N, H * 128])."""
    o = np.asarray(o, np.float64)
    x = o.reshape(o.shape[:-2] + (o.shape[-2] * o.shape[-1],))
    return x @ np.asarray(W_O, np.float64).T

