"""Plain fp64 reference for weight-absorbed MLA decode (numpy).

TEST INFRASTRUCTURE ONLY: see the package docstring.  Slow on purpose and
written for a reader who checks it by eye against the definition below.

What is computed (the absorbed decode attention of DeepSeek-V2/V3 MLA, which
the Huawei Ascend report, "DeepSeek V3/R1 inference deployment best practices
on Ascend servers", uses for decode in section 3.2.1 and section 6.1 and cites
to the DeepSeek-V2 paper):

  Each cached token t of request b is one 576-wide row
      K_t = [c_kv_t (512) | k_pe_t (64)],   V_t = c_kv_t = K_t[0:512]
  shared by every head (section 3.2.1 of that report: all heads share the
  compressed cache).  Query j of request b, head h, is
      q = [q_nope_absorbed[b, j, h] (512) | q_pe[b, j, h] (64)].
  Query j sees keys t = 0 .. n_j - 1 with n_j = L_b - q_len + 1 + j
  (L_b counts the q_len new tokens, already in the cache; the draft token
  j = 1 sees one key more than j = 0).
      s_t = scale * (q . K_t)
      lse = log sum_t exp(s_t)          (natural log of scaled scores)
      out = sum_t exp(s_t - lse) * V_t

Paging: token t of request b is slot t % P of page block_table[b, t // P].

Readings where the pages are silent (each also listed in the design notes):
scale is a parameter (1/sqrt(192) in the workloads); the lse is the natural
log over scaled scores; block-table entries past the last needed page and
slots past L_b in the last page are never touched.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = 576


def visible_keys(L: int, q_len: int, j: int) -> int:
    """Number of keys query j of a request with L cached tokens attends to."""
    return int(L) - int(q_len) + 1 + int(j)


def gather_kv_rows(cache: np.ndarray, bt_row: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Rows [lo, hi) of one request's cache as a dense [hi-lo, 576] fp64 array.

    cache: [num_pages, P, 576] float64, bt_row: the request's block-table row.
    Follows the paging rule literally: token t -> page bt_row[t // P], slot t % P.
    """
    P = cache.shape[1]
    t = np.arange(lo, hi)
    pages = np.asarray(bt_row)[t // P]
    return cache[pages, t % P, :]


def attend_rows(q: np.ndarray, K: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of queries q [..., 576] over rows K [n, 576], V = K[:, :512].

    Returns (out [..., 512], lse [...]).  With n = 0 the result is the empty
    set's: lse = -inf and out = 0 (the neutral element of the merge below).
    """
    lead = q.shape[:-1]
    if K.shape[0] == 0:
        return np.zeros(lead + (D_LATENT,)), np.full(lead, -np.inf)
    s = scale * (q @ K.T)  # [..., n]
    m = s.max(axis=-1, keepdims=True)
    z = np.exp(s - m).sum(axis=-1, keepdims=True)
    lse = m + np.log(z)
    w = np.exp(s - lse)
    out = w @ K[:, :D_LATENT]
    return out, lse[..., 0]


def mla_decode_ref(
    q_nope: np.ndarray,
    q_pe: np.ndarray,
    cache: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
) -> Tuple[np.ndarray, np.ndarray]:
    """The definition, one (request, query) at a time.

    q_nope [B, q_len, H, 512], q_pe [B, q_len, H, 64], cache [num_pages, P, 576]
    (all float64), block_table [B, *] int, seq_lens [B].
    Returns out [B, q_len, H, 512] and lse [B, q_len, H] (float64).
    """
    B, q_len, H, _ = q_nope.shape
    out = np.zeros((B, q_len, H, D_LATENT))
    lse = np.zeros((B, q_len, H))
    for b in range(B):
        L = int(seq_lens[b])
        K_all = gather_kv_rows(cache, block_table[b], 0, L)
        for j in range(q_len):
            n = visible_keys(L, q_len, j)
            q = np.concatenate([q_nope[b, j], q_pe[b, j]], axis=-1)  # [H, 576]
            out[b, j], lse[b, j] = attend_rows(q, K_all[:n], scale)
    return out, lse


def lse_combine_ref(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge per-range results (o_r, lse_r) into the result over the union.

    lse = log sum_r exp(lse_r);  out = sum_r exp(lse_r - lse) * o_r.
    Ranges whose lse is -inf (no keys) contribute nothing; if every range is
    empty the merged lse is -inf and out is 0.
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])  # [R, ...]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])  # [R, ..., 512]
    m = L.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    z = np.exp(L - m_safe).sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(z), -np.inf)
    w = np.where(finite, np.exp(L - np.where(finite, lse, 0.0)), 0.0)  # [R, ...]
    out = (w[..., None] * O).sum(axis=0)
    return out, lse


def mla_decode_split_ref(
    q_nope: np.ndarray,
    q_pe: np.ndarray,
    cache: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
    cuts: Sequence[Sequence[int]],
) -> Tuple[np.ndarray, np.ndarray]:
    """Split-KV form: request b's range [0, L_b) is cut at cuts[b] (sorted interior
    points), each piece is attended separately (keys beyond a query's visible
    count dropped) and the pieces are merged with lse_combine_ref.

    In exact arithmetic this equals mla_decode_ref for any choice of cuts; this is
    the flash-decoding split the Ascend troubleshooting note on decode TPOT jitter
    names in its section 4.2(3).
    """
    B, q_len, H, _ = q_nope.shape
    out = np.zeros((B, q_len, H, D_LATENT))
    lse = np.zeros((B, q_len, H))
    for b in range(B):
        L = int(seq_lens[b])
        bounds = [0] + [int(c) for c in cuts[b]] + [L]
        for j in range(q_len):
            n = visible_keys(L, q_len, j)
            q = np.concatenate([q_nope[b, j], q_pe[b, j]], axis=-1)
            parts_o, parts_l = [], []
            for lo, hi in zip(bounds[:-1], bounds[1:]):
                hi_v = min(hi, n)
                K = gather_kv_rows(cache, block_table[b], lo, max(lo, hi_v))
                o, l = attend_rows(q, K, scale)
                parts_o.append(o)
                parts_l.append(l)
            out[b, j], lse[b, j] = lse_combine_ref(parts_o, parts_l)
    return out, lse


def absorb_query(q_nope128: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """Fold the key up-projection into the query.

    q_nope128 [..., H, 128], W_UK [H, 128, 512] (head h decompresses c_kv to its
    128-wide key part as W_UK[h] @ c_kv).  Returns W_UK[h]^T q_nope_h, [..., H, 512],
    so that q_nope_h . (W_UK[h] c) = (W_UK[h]^T q_nope_h) . c.
    """
    return np.einsum("...hd,hdc->...hc", q_nope128, W_UK)


def mha_unabsorbed_ref(
    q_nope128: np.ndarray,
    q_pe: np.ndarray,
    cache: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    W_UK: np.ndarray,
    W_UV: np.ndarray,
    scale: float,
) -> Tuple[np.ndarray, np.ndarray]:
    """Standard multi-head attention on the decompressed cache (no absorption).

    Per head h: k_{t,h} = [W_UK[h] c_kv_t ; k_pe_t] (192 wide), v_{t,h} = W_UV[h] c_kv_t
    (128 wide), q = [q_nope_h ; q_pe_h] (192 wide), softmax over scale * q.k.
    Returns o [B, q_len, H, 128] and lse [B, q_len, H].
    Weight absorption is an exact algebraic rewrite (the Huawei report's
    abstract lists such equivalent rewrites among its operator techniques and
    sections 3.2.1 and 6.1 apply absorption to decode): o_h must equal
    W_UV[h] @ out_h and lse_h must equal the absorbed form's lse.
    """
    B, q_len, H, dn = q_nope128.shape
    dv = W_UV.shape[1]
    o = np.zeros((B, q_len, H, dv))
    lse = np.zeros((B, q_len, H))
    for b in range(B):
        L = int(seq_lens[b])
        rows = gather_kv_rows(cache, block_table[b], 0, L)
        c_kv, k_pe = rows[:, :D_LATENT], rows[:, D_LATENT:]
        for h in range(H):
            k = np.concatenate([c_kv @ W_UK[h].T, k_pe], axis=1)  # [L, 192]
            v = c_kv @ W_UV[h].T  # [L, 128]
            for j in range(q_len):
                n = visible_keys(L, q_len, j)
                q = np.concatenate([q_nope128[b, j, h], q_pe[b, j, h]])
                s = scale * (k[:n] @ q)
                m = s.max()
                lse[b, j, h] = m + math.log(np.exp(s - m).sum())
                o[b, j, h] = np.exp(s - lse[b, j, h]) @ v[:n]
    return o, lse


def brute_force_ref(
    q_nope: List,
    q_pe: List,
    cache: List,
    block_table: List,
    seq_lens: Sequence[int],
    scale: float,
) -> Tuple[list, list]:
    """Pure-Python loops with the math module only, for tiny inputs.

    Arguments are nested lists (or arrays indexed element by element).  Shares no
    vectorised code with mla_decode_ref; written straight from the definition in
    the module docstring.
    """
    B = len(q_nope)
    q_len = len(q_nope[0])
    H = len(q_nope[0][0])
    P = len(cache[0])
    out = [[[[0.0] * D_LATENT for _ in range(H)] for _ in range(q_len)] for _ in range(B)]
    lse = [[[0.0] * H for _ in range(q_len)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        for j in range(q_len):
            n = L - q_len + 1 + j
            for h in range(H):
                scores = []
                for t in range(n):
                    row = cache[int(block_table[b][t // P])][t % P]
                    acc = 0.0
                    for d in range(D_LATENT):
                        acc += float(q_nope[b][j][h][d]) * float(row[d])
                    for d in range(D_ROPE):
                        acc += float(q_pe[b][j][h][d]) * float(row[D_LATENT + d])
                    scores.append(scale * acc)
                m = max(scores)
                z = 0.0
                for s in scores:
                    z += math.exp(s - m)
                lse_v = m + math.log(z)
                lse[b][j][h] = lse_v
                acc_o = [0.0] * D_LATENT
                for t in range(n):
                    w = math.exp(scores[t] - lse_v)
                    row = cache[int(block_table[b][t // P])][t % P]
                    for d in range(D_LATENT):
                        acc_o[d] += w * float(row[d])
                out[b][j][h] = acc_o
    return out, lse
