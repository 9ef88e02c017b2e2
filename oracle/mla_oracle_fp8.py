"""Plain fp64 reference for absorbed-MLA decode over an FP8 latent cache (numpy).

TEST INFRASTRUCTURE ONLY: see the package docstring.

The pages describe the computation in bf16 and name 8-bit keys and values as
future work (Huawei, "DeepSeek V3/R1 inference deployment best practices on
Ascend servers", section 8 on next steps, the bullet on INT8 KV and fully
INT8 MLA operators; the digest of "Serving LLMs on Huawei CloudMatrix384"
notes, in its description of the Ascend 910 die, that the part has no FP8).
This module fixes the FP8 variant the HIP library implements; every choice
below is a reading, listed with the others in the design notes:

  * cache format: each cached token t holds 576 OCP FP8 E4M3 codes (the
    "fn" encoding: exponent bias 7, no infinities, S.1111.111 is NaN, largest
    finite magnitude 448) and one scale exponent byte e_t in the OCP MX E8M0
    encoding (value 2^(e_t - 127), 255 is NaN).  The token's row is
        K_t = 2^(e_t - 127) * decode(codes_t),   V_t = K_t[0:512];
  * queries arrive in bf16, as in the bf16 path, and are quantized in the
    OCP MXFP8 way: each block of 32 consecutive values of a (request, query
    token, head) row of 576 gets its own exponent f, the smallest integer
    with amax * 2^-f <= 448 (f = 0 for a zero block), limited to the E8M0
    range [-127, 127]; its codes are the nearest E4M3 values of q * 2^-f
    (ties to the even code; limiting f from below keeps the block under 448,
    and bf16 cannot reach the upper limit).  Scaling by a power of two is
    exact, so the only rounding is the final one;
  * attention is then the definition of the bf16 path applied to the
    dequantized rows, in fp64: s_t = scale * (q_deq . K_t), lse = log sum
    exp s_t, out = sum_t exp(s_t - lse) V_t.

The HIP kernel also rounds the softmax weights to E4M3 before the PV product
(the FP8 matrix instruction takes 8-bit operands on both sides).  That is an
approximation of the definition, not part of it; ``fp8_weight_error_rms``
gives the size of its effect, which the parity tests use as the tolerance.
"""
from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np

from .mla_oracle import D_LATENT, D_QK, attend_rows, gather_kv_rows, visible_keys

E4M3_MAX = 448.0
E8M0_BIAS = 127


def e4m3_value(code: int) -> float:
    """The value of one E4M3 ("fn") code, from the format's definition.

    Bit 7 is the sign, bits 6..3 the exponent field E (bias 7), bits 2..0 the
    mantissa M.  E = 0 is subnormal: M/8 * 2^-6; otherwise (1 + M/8) * 2^(E-7).
    E = 15 with M = 7 is NaN (there are no infinities).
    """
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    E = (code >> 3) & 0xF
    M = code & 0x7
    if E == 15 and M == 7:
        return math.nan
    if E == 0:
        return sign * (M / 8.0) * 2.0 ** -6
    return sign * (1.0 + M / 8.0) * 2.0 ** (E - 7)


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes (float64, NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode an array of E4M3 codes to float64."""
    return e4m3_table()[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even code (mantissa LSB 0).

    Written as the definition: among the finite codes, take the one whose
    value is closest to x; on a tie, the one with an even code.  Values whose
    magnitude reaches 464 (half-way to the next power-of-two step beyond 448,
    which the format lacks) have no nearest finite code here and raise.
    Negative zero is returned for negative values that round to zero.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no E4M3 rounding here")
    if (np.abs(x) >= 464.0).any():
        raise ValueError("|x| >= 464 is outside the E4M3 range")
    table = e4m3_table()
    pos_codes = np.arange(0x00, 0x7F)  # +0 .. +448
    pos_vals = table[pos_codes]
    a = np.abs(x).reshape(-1)
    # index of the largest positive value <= a (pos_vals is increasing)
    hi = np.searchsorted(pos_vals, a, side="right")
    lo = np.clip(hi - 1, 0, len(pos_vals) - 1)
    hi = np.clip(hi, 0, len(pos_vals) - 1)
    d_lo = a - pos_vals[lo]
    d_hi = pos_vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (pos_codes[hi] % 2 == 0) & (hi != lo))
    mag = np.where(pick_hi, pos_codes[hi], pos_codes[lo])
    sign = (np.signbit(x.reshape(-1))).astype(np.int64) << 7
    return (mag | sign).astype(np.uint8).reshape(x.shape)


def e8m0_decode(e: np.ndarray) -> np.ndarray:
    """Scale values 2^(e - 127) of E8M0 bytes (255 -> NaN)."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - E8M0_BIAS)
    return np.where(e == 255, np.nan, v)


def query_exponent(amax: float) -> int:
    """Smallest integer f with amax * 2^-f <= 448 (0 for amax == 0).

    Found by walking f from a guess, so the answer is checked against the
    defining inequality itself (power-of-two scaling is exact in fp64).
    """
    amax = float(amax)
    if not (amax >= 0.0) or math.isinf(amax):
        raise ValueError("amax must be finite and >= 0")
    if amax == 0.0:
        return 0
    f = math.frexp(amax / E4M3_MAX)[1] - 2
    while math.ldexp(amax, -f) > E4M3_MAX:
        f += 1
    while math.ldexp(amax, -(f - 1)) <= E4M3_MAX:
        f -= 1
    return f


#: values per query block sharing one exponent (the OCP MX block size)
MX_BLOCK = 32


def quantize_query(q_nope: np.ndarray, q_pe: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantization of the queries.

    q_nope [..., 512] and q_pe [..., 64] (float64 holding bf16 values).
    Returns (codes [..., 576] uint8, f [..., 18] int64): value k of a row is
    about decode(codes[k]) * 2^f[k // 32].
    """
    q = np.concatenate([np.asarray(q_nope, np.float64), np.asarray(q_pe, np.float64)], axis=-1)
    lead = q.shape[:-1]
    nb = D_QK // MX_BLOCK
    blocks = q.reshape(-1, nb, MX_BLOCK)
    codes = np.zeros(blocks.shape, dtype=np.uint8)
    f = np.zeros(blocks.shape[:2], dtype=np.int64)
    for r in range(blocks.shape[0]):
        for k in range(nb):
            fb = min(max(query_exponent(np.abs(blocks[r, k]).max()), -127), 127)
            f[r, k] = fb
            codes[r, k] = e4m3_round(np.clip(np.ldexp(blocks[r, k], -fb), -E4M3_MAX, E4M3_MAX))
    return codes.reshape(lead + (D_QK,)), f.reshape(lead + (nb,))


def dequantize_query(codes: np.ndarray, f: np.ndarray) -> np.ndarray:
    """decode(codes) * 2^f per block, float64 [..., 576]."""
    return np.ldexp(e4m3_decode(codes), np.repeat(np.asarray(f, np.int64), MX_BLOCK, axis=-1))


def dequantize_cache(codes: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """Cached rows as float64: codes [num_pages, P, 576] uint8, exps [num_pages, P] uint8."""
    return e4m3_decode(codes) * e8m0_decode(exps)[..., None]


def mla_decode_fp8_ref(
    q_nope: np.ndarray,
    q_pe: np.ndarray,
    cache_codes: np.ndarray,
    cache_exps: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
) -> Tuple[np.ndarray, np.ndarray]:
    """The FP8 variant's definition: quantize the queries, dequantize the cache,
    then the attention of the bf16 path in fp64.

    Returns out [B, q_len, H, 512] and lse [B, q_len, H] (float64).
    """
    codes, f = quantize_query(q_nope, q_pe)
    q = dequantize_query(codes, f)  # [B, q_len, H, 576]
    cache = dequantize_cache(cache_codes, cache_exps)
    B, q_len, H, _ = q.shape
    out = np.zeros((B, q_len, H, D_LATENT))
    lse = np.zeros((B, q_len, H))
    for b in range(B):
        L = int(seq_lens[b])
        K_all = gather_kv_rows(cache, block_table[b], 0, L)
        for j in range(q_len):
            n = visible_keys(L, q_len, j)
            out[b, j], lse[b, j] = attend_rows(q[b, j], K_all[:n], scale)
    return out, lse


#: E4M3 keeps 3 mantissa bits: a normal value x = 2^(k + phi) (0 <= phi < 1)
#: lies on a grid of step 2^(k - 3), so rounding to nearest changes it by at
#: most half a step, 2^(-4 - phi) of itself.  An error spread evenly over
#: +-half a step has a root mean square of step / sqrt(12); relative to x that
#: is 2^(-3 - phi) / sqrt(12), largest (2^-4 / sqrt(3)) at the bottom of a binade:
E4M3_REL_RMS = 2.0 ** -4 / math.sqrt(3.0)
#: and, averaged over where x falls inside its binade (phi uniform, as for the
#: kernel's scaled weights, whose log2 has no preferred fractional part), the
#: root of the mean of 2^(-6 - 2 phi) / 12 = 2^-3 / sqrt(12) * sqrt(3 / (8 ln 2)).
E4M3_REL_RMS_AVG = 2.0 ** -3 / math.sqrt(12.0) * math.sqrt(3.0 / (8.0 * math.log(2.0)))


def fp8_weight_error_rms(
    q_nope: np.ndarray,
    q_pe: np.ndarray,
    cache_codes: np.ndarray,
    cache_exps: np.ndarray,
    block_table: np.ndarray,
    seq_lens: Sequence[int],
    scale: float,
    weight_exp: int = 6,
) -> np.ndarray:
    """Root-mean-square size of the output error that rounding the softmax
    weights to E4M3 causes, per output element [B, q_len, H, 512].

    Model: before rounding, weight w_t of the exact softmax is scaled to
        a_t = w_t / w_max * 2^weight_exp * 2^(e_t - e_max)
    (the row's largest weight lands at 2^weight_exp for a token with the
    largest scale exponent e_max of the request).  A normal a_t (>= 2^-6) is
    rounded with independent relative error of rms E4M3_REL_RMS_AVG (the
    uniform-rounding-noise rms of the E4M3 grid averaged over the position
    inside the binade: the kernel puts each tile's largest weight at a
    position inside [2^6, 2^7) set by the scores, not at the binade's
    bottom); a subnormal one with absolute error of rms
    min(2^-10 / sqrt(3), a_t) (the subnormal step is 2^-9; values below half
    a step round to zero).  Back in weight units the error is
    err_t = that / (a_t / w_t), and the output error of element d is
    sqrt(sum_t err_t^2 V_td^2).
    """
    codes, f = quantize_query(q_nope, q_pe)
    q = dequantize_query(codes, f)
    cache = dequantize_cache(cache_codes, cache_exps)
    B, q_len, H, _ = q.shape
    P = cache.shape[1]
    rms = np.zeros((B, q_len, H, D_LATENT))
    for b in range(B):
        L = int(seq_lens[b])
        K_all = gather_kv_rows(cache, block_table[b], 0, L)
        t = np.arange(L)
        e_all = np.asarray(cache_exps)[np.asarray(block_table[b])[t // P], t % P].astype(np.int64)
        for j in range(q_len):
            n = visible_keys(L, q_len, j)
            if n <= 0:
                continue
            K = K_all[:n]
            # the largest exponent of the whole request (masked keys included)
            # bounds the one any piece of it scales by
            gain = np.ldexp(1.0, weight_exp + e_all[:n] - e_all.max())[None, :]  # [1, n]
            s = scale * (q[b, j] @ K.T)  # [H, n]
            w = np.exp(s - s.max(axis=-1, keepdims=True))
            w /= w.sum(axis=-1, keepdims=True)
            a = w / w.max(axis=-1, keepdims=True) * gain
            err_a = np.where(a >= 2.0**-6, E4M3_REL_RMS_AVG * a, np.minimum(2.0**-10 / math.sqrt(3.0), a))
            err = err_a * (w / np.where(a > 0, a, 1.0))
            rms[b, j] = np.sqrt((err**2) @ (K[:, :D_LATENT] ** 2))
    return rms
