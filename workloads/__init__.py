"""Seeded synthetic inputs for absorbed-MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the fp64 oracle (through the tests) and the HIP
path (through the tests and the benchmark) take their inputs from here, so the
two sides always see identical bits.

Workload shapes come from the pages:

* H = 128 heads, a 512-wide absorbed latent part and a 64-wide rope part per
  query head, 576 bf16 values per cached token (Huawei, "DeepSeek V3/R1
  inference deployment best practices on Ascend servers", section 7.2, the MLA
  time model with its (576 + 512) x 128 terms; section 3.1.1 for the BF16
  KV cache).
* One MTP draft token, i.e. two query tokens per request (same report,
  section 5.3 and the x2 factor in section 7.2); 3 and 7 draft tokens for
  the longer-draft workloads (the digest of the LMSYS post on serving
  DeepSeek-V4-Pro on H20 runs 7 draft tokens; the CloudMatrix384 digest
  speculates a single token).
* A mixed batch of 20K-token (40%) and 400-token (60%) requests (Ascend
  troubleshooting note on decode TPOT jitter, section 5.2, the random mixed
  data set).

Generation recipe (fixed draw order, ``numpy.random.default_rng(seed)``):
  1. sequence lengths (only the "mtp" configs draw them),
  2. a shuffle of the request order,
  3. a permutation of all pages, dealt to the requests in order,
  4. q_nope_absorbed, 5. q_pe, 6. the paged cache;
values are float32 N(0, 1) rounded to bf16 (round-to-nearest-even).
``num_pages`` is the exact number of pages the requests need; unused
block-table entries hold -1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE  # 576

#: The five named workloads.  ``lens`` is either a fixed list or a rule.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(seed=1, batch=2, heads=16, q_len=1, page=16, lens=[37, 100]),
    "dsv3": dict(seed=2, batch=32, heads=128, q_len=1, page=64, lens=[4096] * 32),
    "mtp": dict(seed=3, batch=64, heads=128, q_len=2, page=64, lens=("uniform", 1024, 8192)),
    # 40% of 64 = 25.6 requests, rounded to 26 long and 38 short.
    "mixed": dict(seed=4, batch=64, heads=128, q_len=1, page=64, lens=[20480] * 26 + [400] * 38),
    "long": dict(seed=5, batch=1, heads=128, q_len=1, page=64, lens=[131072]),
    # More draft tokens (3 and 7 drafts: 4 and 8 query tokens per request),
    # the same 16384 query rows as "mtp" over fewer requests.
    "mtp4": dict(seed=6, batch=32, heads=128, q_len=4, page=64, lens=("uniform", 1024, 8192)),
    "mtp8": dict(seed=7, batch=16, heads=128, q_len=8, page=64, lens=("uniform", 1024, 8192)),
}
CONFIG_ORDER = ["tiny", "dsv3", "mtp", "mixed", "long"]
#: workloads beyond the five headline ones (more draft tokens)
EXTRA_CONFIGS = ["mtp4", "mtp8"]


def softmax_scale_default() -> float:
    """1/sqrt(192) rounded to float32: the value the library receives.

    192 = 128 (no-rope part) + 64 (rope part) is the per-head query/key width of
    the unabsorbed attention; absorption changes the dot-product width to 576
    but not the scale.
    """
    return float(np.float32(1.0 / np.sqrt(192.0)))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even) and return the raw uint16 bits.

    NaN inputs stay NaN (a quiet NaN pattern).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    r = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to float64 exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class MLAInputs:
    """One batch of decode inputs.  bf16 tensors are held as raw uint16 bits."""

    name: str
    batch: int
    heads: int
    q_len: int
    page: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, bt_stride], -1 padded
    num_pages: int
    q_nope: np.ndarray  # uint16 [B, q_len, H, 512]
    q_pe: np.ndarray  # uint16 [B, q_len, H, 64]
    cache: np.ndarray  # uint16 [num_pages, page, 576]
    softmax_scale: float = field(default_factory=softmax_scale_default)

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    # float64 views for the oracle
    def q_nope_f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.q_nope)

    def q_pe_f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.q_pe)

    def cache_f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.cache)

    def to_torch(self, device: str = "cpu") -> dict:
        """Torch tensors (bf16 views of the same bits) for the HIP path."""
        import torch

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

        return dict(
            q_nope=bf16(self.q_nope),
            q_pe=bf16(self.q_pe),
            cache=bf16(self.cache),
            block_table=torch.from_numpy(np.ascontiguousarray(self.block_table)).to(device),
            seq_lens=torch.from_numpy(np.ascontiguousarray(self.seq_lens)).to(device),
        )


def pages_needed(lens: Sequence[int], page: int) -> List[int]:
    return [-(-int(L) // page) for L in lens]


def make_inputs(
    batch: int,
    heads: int,
    q_len: int,
    page: int,
    lens: Sequence[int] | tuple,
    seed: int,
    name: str = "custom",
    extra_pages: int = 0,
    draw_values: bool = True,
) -> MLAInputs:
    """Draw one seeded batch following the fixed recipe in the module docstring.

    ``lens`` is a list of per-request lengths or ``("uniform", lo, hi)`` for
    integer lengths drawn uniformly from [lo, hi] (both ends included).
    ``extra_pages`` appends unreferenced pages after the referenced ones (their
    contents are drawn too, and callers may poison them).
    """
    rng = np.random.default_rng(seed)
    seq_lens, block_table, num_pages = _draw_layout(rng, batch, page, lens, extra_pages)
    if draw_values:
        q_nope = to_bf16_bits(rng.standard_normal((batch, q_len, heads, D_LATENT), dtype=np.float32))
        q_pe = to_bf16_bits(rng.standard_normal((batch, q_len, heads, D_ROPE), dtype=np.float32))
        cache = to_bf16_bits(rng.standard_normal((num_pages, page, D_QK), dtype=np.float32))
    else:
        q_nope = np.zeros((batch, q_len, heads, D_LATENT), np.uint16)
        q_pe = np.zeros((batch, q_len, heads, D_ROPE), np.uint16)
        cache = np.zeros((num_pages, page, D_QK), np.uint16)
    return MLAInputs(
        name=name,
        batch=batch,
        heads=heads,
        q_len=q_len,
        page=page,
        seq_lens=seq_lens,
        block_table=block_table,
        num_pages=num_pages,
        q_nope=q_nope,
        q_pe=q_pe,
        cache=cache,
    )


def _draw_layout(rng, batch: int, page: int, lens, extra_pages: int):
    """Steps 1-3 of the recipe: lengths, request order, page permutation."""
    if isinstance(lens, tuple) and lens and lens[0] == "uniform":
        _, lo, hi = lens
        base = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    else:
        base = np.asarray(list(lens), dtype=np.int64)
        if base.shape[0] != batch:
            raise ValueError("len(lens) must equal batch")
    order = rng.permutation(batch)
    seq_lens = base[order].astype(np.int32)

    npg = pages_needed(seq_lens, page)
    used = int(sum(npg))
    num_pages = used + int(extra_pages)
    perm = rng.permutation(used).astype(np.int32)
    bt_stride = max(1, max(npg) if npg else 1)
    block_table = np.full((batch, bt_stride), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        block_table[b, :n] = perm[off : off + n]
        off += n
    return seq_lens, block_table, num_pages


def make_config(name: str, seed: Optional[int] = None) -> MLAInputs:
    """The named workload with its own seed (or an override)."""
    c = CONFIGS[name]
    return make_inputs(
        batch=c["batch"],
        heads=c["heads"],
        q_len=c["q_len"],
        page=c["page"],
        lens=c["lens"],
        seed=c["seed"] if seed is None else seed,
        name=name,
    )


def config_lens(name: str) -> np.ndarray:
    """Sequence lengths of a named workload without drawing the large tensors."""
    c = CONFIGS[name]
    x = make_inputs(c["batch"], c["heads"], c["q_len"], c["page"], c["lens"], c["seed"], name, draw_values=False)
    return x.seq_lens


def poison_tails(x: MLAInputs, value_bits: int = 0x7FC0) -> None:
    """Fill the unused slots of every request's last page with NaN (in place)."""
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        n = -(-L // x.page)
        tail = L - (n - 1) * x.page
        if tail < x.page:
            x.cache[x.block_table[b, n - 1], tail:, :] = value_bits


def poison_unreferenced(x: MLAInputs, value_bits: int = 0x7FC0) -> None:
    """Fill every page no request references with NaN (in place)."""
    ref = np.zeros(x.num_pages, dtype=bool)
    for b in range(x.batch):
        n = -(-int(x.seq_lens[b]) // x.page)
        ref[x.block_table[b, :n]] = True
    x.cache[~ref] = value_bits


# ---------------------------------------------------------------------------
# FP8 latent cache
# ---------------------------------------------------------------------------
#: Cache values are drawn as N(0, 1) and stored as E4M3 codes of 64 x (so the
#: largest |x| the draw keeps, 7, maps to 448); the token's E8M0 scale byte is
#: 121 + k with k uniform in {-2, ..., 2}, so token t's row is about 2^k x:
#: token magnitudes spread over a factor 16, as a per-token scale is there for.
FP8_CODE_GAIN = 64.0
FP8_CLIP = 7.0
FP8_EXP_CENTER = 121
FP8_EXP_SPREAD = 2


@dataclass
class MLAInputsFP8:
    """One batch of decode inputs over an FP8 cache (queries as bf16 bits)."""

    name: str
    batch: int
    heads: int
    q_len: int
    page: int
    seq_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, bt_stride], -1 padded
    num_pages: int
    q_nope: np.ndarray  # uint16 [B, q_len, H, 512]
    q_pe: np.ndarray  # uint16 [B, q_len, H, 64]
    cache_codes: np.ndarray  # uint8 [num_pages, page, 576], E4M3
    cache_exps: np.ndarray  # uint8 [num_pages, page], E8M0
    softmax_scale: float = field(default_factory=softmax_scale_default)

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    def q_nope_f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.q_nope)

    def q_pe_f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.q_pe)

    def to_torch(self, device: str = "cpu") -> dict:
        """Torch tensors of the same bits for the HIP path."""
        import torch

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

        return dict(
            q_nope=bf16(self.q_nope),
            q_pe=bf16(self.q_pe),
            cache_codes=torch.from_numpy(np.ascontiguousarray(self.cache_codes)).to(device),
            cache_exps=torch.from_numpy(np.ascontiguousarray(self.cache_exps)).to(device),
            block_table=torch.from_numpy(np.ascontiguousarray(self.block_table)).to(device),
            seq_lens=torch.from_numpy(np.ascontiguousarray(self.seq_lens)).to(device),
        )


def e4m3_codes_of(x: np.ndarray) -> np.ndarray:
    """E4M3 codes of float32 values via torch's float8_e4m3fn conversion (a
    library routine; |x| must stay within 448)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def make_inputs_fp8(
    batch: int,
    heads: int,
    q_len: int,
    page: int,
    lens: Sequence[int] | tuple,
    seed: int,
    name: str = "custom",
    extra_pages: int = 0,
) -> MLAInputsFP8:
    """Draw one seeded FP8 batch: steps 1-5 of the bf16 recipe (lengths,
    order, pages, q_nope, q_pe), then 6. cache values N(0, 1) float32, clipped
    to +-FP8_CLIP and stored as codes of FP8_CODE_GAIN * x, 7. per-token scale
    bytes FP8_EXP_CENTER + k, k uniform in [-FP8_EXP_SPREAD, FP8_EXP_SPREAD]."""
    rng = np.random.default_rng(seed)
    seq_lens, block_table, num_pages = _draw_layout(rng, batch, page, lens, extra_pages)
    q_nope = to_bf16_bits(rng.standard_normal((batch, q_len, heads, D_LATENT), dtype=np.float32))
    q_pe = to_bf16_bits(rng.standard_normal((batch, q_len, heads, D_ROPE), dtype=np.float32))
    x = rng.standard_normal((num_pages, page, D_QK), dtype=np.float32)
    np.clip(x, -FP8_CLIP, FP8_CLIP, out=x)
    x *= np.float32(FP8_CODE_GAIN)
    codes = e4m3_codes_of(x)
    k = rng.integers(-FP8_EXP_SPREAD, FP8_EXP_SPREAD + 1, size=(num_pages, page))
    exps = (FP8_EXP_CENTER + k).astype(np.uint8)
    return MLAInputsFP8(
        name=name,
        batch=batch,
        heads=heads,
        q_len=q_len,
        page=page,
        seq_lens=seq_lens,
        block_table=block_table,
        num_pages=num_pages,
        q_nope=q_nope,
        q_pe=q_pe,
        cache_codes=codes,
        cache_exps=exps,
    )


def make_config_fp8(name: str, seed: Optional[int] = None) -> MLAInputsFP8:
    """A named workload's shapes and seed with an FP8 cache."""
    c = CONFIGS[name]
    return make_inputs_fp8(
        batch=c["batch"],
        heads=c["heads"],
        q_len=c["q_len"],
        page=c["page"],
        lens=c["lens"],
        seed=c["seed"] if seed is None else seed,
        name=name,
    )


def poison_tails_fp8(x: MLAInputsFP8) -> None:
    """NaN codes (0x7F) and NaN scale bytes (255) in the unused slots of every
    request's last page (in place)."""
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        n = -(-L // x.page)
        tail = L - (n - 1) * x.page
        if tail < x.page:
            x.cache_codes[x.block_table[b, n - 1], tail:, :] = 0x7F
            x.cache_exps[x.block_table[b, n - 1], tail:] = 255


def poison_unreferenced_fp8(x: MLAInputsFP8) -> None:
    """NaN codes and scale bytes in every page no request references (in place)."""
    ref = np.zeros(x.num_pages, dtype=bool)
    for b in range(x.batch):
        n = -(-int(x.seq_lens[b]) // x.page)
        ref[x.block_table[b, :n]] = True
    x.cache_codes[~ref] = 0x7F
    x.cache_exps[~ref] = 255


# ---------------------------------------------------------------------------
# Prolog / epilog inputs (the steps around the decode attention)
# ---------------------------------------------------------------------------
ROPE_THETA = 10000.0


@dataclass
class PrologInputs:
    """One decode step's inputs to the prolog and the weights of the epilog.

    bf16 tensors as raw uint16 bits; the RoPE table as float32."""

    batch: int
    q_len: int
    heads: int
    seq_lens: np.ndarray  # int32 [B] (the q_len new tokens included)
    q_nope128: np.ndarray  # uint16 [B, q_len, H, 128]
    q_pe_raw: np.ndarray  # uint16 [B, q_len, H, 64]
    w_uk_t: np.ndarray  # uint16 [H, 512, 128]: element [h, c, d] = W_UK[h][d][c]
    c_kv_raw: np.ndarray  # uint16 [B, q_len, 512]
    kv_norm_w: np.ndarray  # uint16 [512]
    k_pe_raw: np.ndarray  # uint16 [B, q_len, 64]
    rope_cos_sin: np.ndarray  # float32 [max_pos, 64]: cos of the 32 pair angles, then their sin
    w_uv: np.ndarray  # uint16 [H, 128, 512]
    w_o: Optional[np.ndarray] = None  # uint16 [hidden, H * 128] (drawn when hidden > 0)
    rms_eps: float = 1e-6

    def w_uk_f64(self) -> np.ndarray:
        """W_UK [H, 128, 512] as float64."""
        return np.ascontiguousarray(bf16_bits_to_f64(self.w_uk_t).transpose(0, 2, 1))


def rope_cos_sin_table(max_pos: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Plain RoPE constants of the model, [max_pos, 64] float32: pair i of
    position p turns by p * theta^(-2i/64); cos of the 32 angles, then sin."""
    inv = theta ** (-np.arange(0, D_ROPE, 2, dtype=np.float64) / D_ROPE)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_prolog_inputs(
    batch: int, q_len: int, heads: int, seq_lens: Sequence[int], seed: int, hidden: int = 0
) -> PrologInputs:
    """Draw order: q_nope (128 wide), q_pe, W_UK^T, c_kv, the norm weight, k_pe,
    W_UV, then (hidden > 0) the output projection W_O [hidden, H * 128]; values
    N(0, 1) except the weights (N(0, 1/sqrt(fan-in))) and the norm weight
    (1 + 0.1 N(0, 1)); all rounded to bf16.  DeepSeek-V3's hidden size is 7168."""
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q_nope = to_bf16_bits(n(batch, q_len, heads, 128))
    q_pe = to_bf16_bits(n(batch, q_len, heads, D_ROPE))
    w_uk_t = to_bf16_bits(n(heads, D_LATENT, 128) / np.float32(np.sqrt(128.0)))
    c_kv = to_bf16_bits(n(batch, q_len, D_LATENT))
    w = to_bf16_bits(np.float32(1.0) + np.float32(0.1) * n(D_LATENT))
    k_pe = to_bf16_bits(n(batch, q_len, D_ROPE))
    w_uv = to_bf16_bits(n(heads, 128, D_LATENT) / np.float32(np.sqrt(float(D_LATENT))))
    w_o = to_bf16_bits(n(hidden, heads * 128) / np.float32(np.sqrt(heads * 128.0))) if hidden > 0 else None
    lens = np.asarray(seq_lens, np.int32)
    return PrologInputs(
        batch=batch, q_len=q_len, heads=heads, seq_lens=lens, q_nope128=q_nope, q_pe_raw=q_pe, w_uk_t=w_uk_t,
        c_kv_raw=c_kv, kv_norm_w=w, k_pe_raw=k_pe, rope_cos_sin=rope_cos_sin_table(int(lens.max()) + 1), w_uv=w_uv,
        w_o=w_o,
    )
