"""The prolog (absorbed query, RoPE, RMSNorm, cache append) and the epilog (value
up-projection, output projection) on an MI355X, through the C ABI, against the fp64 oracle.

Bars, derived from the arithmetic (fp32 inside the kernels, bf16 results):
  * a bf16 result r of an exact value v made of terms t_i (a dot product, a
    rotation) obeys |r - v| <= 2^-8 |v| + 2^-15 sum|t_i|: half a bf16 ulp of
    rounding plus at most 512 * 2^-24 of the terms' magnitudes for the fp32
    sums; the RMSNorm rows take 2^-14 |v| for the sum of squares and the
    reciprocal square root;
  * the up-projection rounds its fp32 input to bf16 (2^-9 per term) before the
    MFMA: |r - v| <= 2^-8 |v| + 2^-8 sum|t_i|, and relative L2 <= 5e-3;
  * the output projection sums K = H * 128 products in fp32 (MFMA chains, then
    the slices' partials): |r - v| <= 2^-8 |v| + K 2^-24 sum|t_i|, and
    relative L2 <= 5e-3;
  * FP8 rows: the E8M0 byte within one of the oracle's (the bf16 row may differ
    in its last bit), the decoded row within one E4M3 step (2^-3 relative, or
    the subnormal step) of the oracle's, and >= 98% of the codes bit-equal;
  * rows the prolog does not write stay bit-identical.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from oracle.mla_oracle_fp8 import e4m3_decode  # noqa: E402
from oracle.mla_prolog_oracle import (  # noqa: E402
    append_ref,
    bf16_round,
    o_project_ref,
    prolog_ref,
    quantize_row_fp8,
    up_project_ref,
)
from tests import test_gpu_fp8 as t8  # noqa: E402
from tests import test_gpu_parity as t16  # noqa: E402
from workloads import (  # noqa: E402
    CONFIGS,
    bf16_bits_to_f64,
    make_config,
    make_config_fp8,
    make_inputs,
    make_inputs_fp8,
    make_prolog_inputs,
    to_bf16_bits,
)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def bf16_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def bits_of(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_prolog(pi, cache, scales, block_table, dev, table=None):
    """Run mla_prolog on copies of the cache; returns (q_abs bits, q_pe bits,
    cache after, scales after)."""
    cs = pi.rope_cos_sin if table is None else table
    c = bf16_dev(cache, dev) if cache.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(cache)).to(dev)
    s = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales)).to(dev)
    qa, qp = mla.mla_prolog(
        bf16_dev(pi.q_nope128, dev), bf16_dev(pi.q_pe_raw, dev), bf16_dev(pi.w_uk_t, dev), bf16_dev(pi.c_kv_raw, dev),
        bf16_dev(pi.kv_norm_w, dev), pi.rms_eps, bf16_dev(pi.k_pe_raw, dev), torch.from_numpy(cs).to(dev),
        torch.from_numpy(pi.seq_lens).to(dev), torch.from_numpy(np.ascontiguousarray(block_table)).to(dev), c, s,
    )
    torch.cuda.synchronize()
    c_out = bits_of(c) if cache.dtype == np.uint16 else c.cpu().numpy()
    return bits_of(qa), bits_of(qp), c_out, (None if s is None else s.cpu().numpy())


def oracle_prolog(pi, table=None):
    cs = (pi.rope_cos_sin if table is None else table).astype(np.float64)
    return prolog_ref(
        bf16_bits_to_f64(pi.q_nope128), bf16_bits_to_f64(pi.q_pe_raw), pi.w_uk_f64(), bf16_bits_to_f64(pi.c_kv_raw),
        bf16_bits_to_f64(pi.kv_norm_w), pi.rms_eps, bf16_bits_to_f64(pi.k_pe_raw), cs[:, :32], cs[:, 32:],
        pi.seq_lens,
    )


def term_sums(pi, table=None):
    """sum|t_i| of every q_abs element and every rotated q_pe / k_pe element."""
    cs = (pi.rope_cos_sin if table is None else table).astype(np.float64)
    qa = np.einsum("bjhd,hdc->bjhc", np.abs(bf16_bits_to_f64(pi.q_nope128)), np.abs(pi.w_uk_f64()))
    L = pi.seq_lens.astype(np.int64)[:, None] - pi.q_len + np.arange(pi.q_len)[None, :]
    c, s = np.abs(cs[L, :32]), np.abs(cs[L, 32:])

    def rot(x):
        a, b = np.abs(x[..., 0::2]), np.abs(x[..., 1::2])
        cc, ss = (c[:, :, None, :], s[:, :, None, :]) if x.ndim == 4 else (c, s)
        out = np.empty_like(x)
        out[..., 0::2] = a * cc + b * ss
        out[..., 1::2] = a * ss + b * cc
        return out

    return qa, rot(bf16_bits_to_f64(pi.q_pe_raw)), rot(bf16_bits_to_f64(pi.k_pe_raw))


def check_bf16(bits, exact, terms, rel_terms, what):
    got = bf16_bits_to_f64(bits)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - exact)
    bar = 2.0**-8 * np.abs(exact) + rel_terms * terms
    # an exact zero (a zero row) must come out zero
    worst = float(np.max(np.divide(err, bar, out=np.where(err > 0, np.inf, 0.0), where=bar > 0)))
    same = float(np.mean(got == bf16_round(exact)))
    print(f"{what}: max-abs {err.max():.3e} worst/bar {worst:.3f} bit-equal to rounded oracle {same:.4f}", flush=True)
    assert worst <= 1.0, f"{what}: an element is {worst:.2f}x past its bar"
    return same


def check_rows_bf16(cache_after, cache_before, pi, block_table, rows, what, table=None):
    """New rows within the bar, every other cache element bit-identical."""
    page = cache_before.shape[1]
    written = np.zeros(cache_before.shape[:2], bool)
    for b in range(pi.batch):
        for j in range(pi.q_len):
            t = int(pi.seq_lens[b]) - pi.q_len + j
            written[int(block_table[b, t // page]), t % page] = True
    assert np.array_equal(cache_after[~written], cache_before[~written]), f"{what}: rows outside the new tokens changed"
    ref = append_ref(np.zeros(cache_before.shape), block_table, pi.seq_lens, rows)
    # the terms behind each element: |v| for the RMSNorm part, the rotation's
    # |x0 c| + |x1 s| for the RoPE part
    _, _, t_kpe = term_sums(pi, table)
    terms = np.concatenate([np.abs(rows[..., :512]), t_kpe], axis=-1)
    tref = append_ref(np.zeros(cache_before.shape), block_table, pi.seq_lens, terms)
    got = cache_after[written]
    exact = ref[written]
    same = check_bf16(got, exact, tref[written], 2.0**-13, what)
    assert same >= 0.98, f"{what}: only {same:.3f} of the row elements are bit-equal"


def check_rows_fp8(codes_after, exps_after, codes_before, exps_before, pi, block_table, rows, what):
    page = codes_before.shape[1]
    written = np.zeros(codes_before.shape[:2], bool)
    for b in range(pi.batch):
        for j in range(pi.q_len):
            t = int(pi.seq_lens[b]) - pi.q_len + j
            written[int(block_table[b, t // page]), t % page] = True
    assert np.array_equal(codes_after[~written], codes_before[~written]), f"{what}: codes outside the new rows changed"
    assert np.array_equal(exps_after[~written], exps_before[~written]), f"{what}: scales outside the new rows changed"
    q = [quantize_row_fp8(r) for r in rows.reshape(-1, 576)]
    ref_codes = np.stack([c for c, _ in q]).reshape(rows.shape)
    ref_exps = np.array([e for _, e in q], np.int64).reshape(rows.shape[:2])
    rc = append_ref(np.zeros(codes_before.shape, np.uint8), block_table, pi.seq_lens, ref_codes)[written]
    re_ = append_ref(np.zeros(exps_before.shape, np.int64), block_table, pi.seq_lens, ref_exps)[written]
    gc, ge = codes_after[written], exps_after[written].astype(np.int64)
    assert np.all(np.abs(ge - re_) <= 1), f"{what}: an E8M0 byte is off by more than one"
    gv = np.ldexp(e4m3_decode(gc), (ge - 127)[:, None])
    rv = np.ldexp(e4m3_decode(rc), (re_ - 127)[:, None])
    # two nearest-even roundings of values one bf16 ulp apart: at most one
    # E4M3 step at the coarser of the two scales (one subnormal step below 2^-6)
    bar = 2.0**-3 * np.maximum(np.abs(rv), np.abs(gv)) + np.ldexp(1.0, (np.maximum(ge, re_) - 127 - 9))[:, None]
    worst = float(np.max(np.abs(gv - rv) / bar))
    same = float(np.mean(gc == rc))
    print(f"{what}: scales equal {np.mean(ge == re_):.4f} codes bit-equal {same:.4f} worst/bar {worst:.3f}", flush=True)
    assert worst <= 1.0, f"{what}: a decoded element is {worst:.2f}x past one E4M3 step"
    assert same >= 0.98, f"{what}: only {same:.3f} of the codes are bit-equal"


def check_prolog_outputs(pi, qa, qp, table=None, what=""):
    q_abs, q_pe, rows = oracle_prolog(pi, table)
    t_qa, t_qp, _ = term_sums(pi, table)
    check_bf16(qa, q_abs, t_qa, 2.0**-15, f"{what} q_nope_absorbed")
    check_bf16(qp, q_pe, t_qp, 2.0**-15, f"{what} q_pe")
    return rows


# ---- small cases: several heads, pages crossed by the new tokens, ragged batches ----------

SMALL = [
    # (batch, heads, q_len, page, lens)
    (3, 16, 2, 16, [5, 17, 40]),
    (1, 1, 1, 16, [1]),
    (2, 128, 1, 64, [64, 65]),
    (5, 8, 4, 16, [4, 16, 19, 33, 100]),
    (37, 2, 1, 16, list(range(1, 38))),  # 37 query rows: a ragged 32-row block
    (70, 4, 2, 16, list(range(2, 72))),  # 140 query rows: two 128-row chunks; 4 heads, so each
                                         # per-token workgroup appends 32 or 3 tokens
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}q{c[2]}p{c[3]}")
def test_prolog_small_bf16(dev, case):
    B, H, q, page, lens = case
    x = make_inputs(B, H, q, page, lens, seed=11)
    pi = make_prolog_inputs(B, q, H, x.seq_lens, seed=12)
    qa, qp, c_after, _ = run_prolog(pi, x.cache, None, x.block_table, dev)
    rows = check_prolog_outputs(pi, qa, qp, what=f"bf16 {case[:4]}")
    check_rows_bf16(c_after, x.cache, pi, x.block_table, rows, f"bf16 {case[:4]} rows")


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}H{c[1]}q{c[2]}p{c[3]}")
def test_prolog_small_fp8(dev, case):
    B, H, q, page, lens = case
    x = make_inputs_fp8(B, H, q, page, lens, seed=13)
    pi = make_prolog_inputs(B, q, H, x.seq_lens, seed=14)
    qa, qp, c_after, s_after = run_prolog(pi, x.cache_codes, x.cache_exps, x.block_table, dev)
    rows = check_prolog_outputs(pi, qa, qp, what=f"fp8 {case[:4]}")
    check_rows_fp8(c_after, s_after, x.cache_codes, x.cache_exps, pi, x.block_table, rows, f"fp8 {case[:4]} rows")


def test_prolog_zero_row_and_wide_range(dev):
    """An all-zero c_kv / k_pe row (RMSNorm of zero with eps > 0 is zero; the FP8
    byte is 127) and rows scaled by 2^-100 and 2^+100 (RMSNorm removes the
    scale; k_pe keeps it, so the E8M0 byte moves with it)."""
    B, H, q, page, lens = 3, 4, 1, 16, [3, 20, 33]
    x = make_inputs_fp8(B, H, q, page, lens, seed=15)
    pi = make_prolog_inputs(B, q, H, x.seq_lens, seed=16)
    ckv, kpe = bf16_bits_to_f64(pi.c_kv_raw), bf16_bits_to_f64(pi.k_pe_raw)
    ckv[0], kpe[0] = 0.0, 0.0
    ckv[1] *= 2.0**-100
    kpe[1] *= 2.0**-100
    ckv[2] *= 2.0**100
    kpe[2] *= 2.0**100
    pi = dataclasses.replace(pi, c_kv_raw=to_bf16_bits(ckv.astype(np.float32)), k_pe_raw=to_bf16_bits(kpe.astype(np.float32)))
    qa, qp, c_after, s_after = run_prolog(pi, x.cache_codes, x.cache_exps, x.block_table, dev)
    rows = check_prolog_outputs(pi, qa, qp, what="fp8 range")
    check_rows_fp8(c_after, s_after, x.cache_codes, x.cache_exps, pi, x.block_table, rows, "fp8 range rows")
    t = int(x.seq_lens[0]) - 1
    slot = int(x.block_table[0, t // page]), t % page
    assert s_after[slot] == 127 and not np.any(c_after[slot] & 0x7F)  # +-0 (a rotation of zeros may give -0)
    xb = make_inputs(B, H, q, page, lens, seed=15)
    _, _, cb_after, _ = run_prolog(pi, xb.cache, None, xb.block_table, dev)
    check_rows_bf16(cb_after, xb.cache, pi, xb.block_table, rows, "bf16 range rows")


def test_prolog_positions_outside_the_table_and_pages(dev):
    """A position past the RoPE table gives NaN q_pe and writes nothing; a new
    token whose page id is outside [0, num_pages) writes nothing; the other
    tokens are unaffected."""
    B, H, q, page, lens = 3, 8, 1, 16, [10, 30, 50]
    x = make_inputs(B, H, q, page, lens, seed=17)
    pi = make_prolog_inputs(B, q, H, x.seq_lens, seed=18)
    table = pi.rope_cos_sin[:40]  # positions 9 and 29 fit, 49 does not
    i10, i30, i50 = (int(np.flatnonzero(x.seq_lens == L)[0]) for L in lens)  # the draw permutes the requests
    bt = x.block_table.copy()
    bt[i30, (30 - 1) // page] = x.num_pages + 5  # the 30-token request's new token lands on no page
    qa, qp, c_after, _ = run_prolog(pi, x.cache, None, bt, dev, table=table)
    assert np.all(np.isnan(bf16_bits_to_f64(qp[i50]))), "a position past the table must give NaN"
    assert np.all(np.isfinite(bf16_bits_to_f64(qp[[i10, i30]])))
    k = [i10]
    ok = dataclasses.replace(pi, batch=1, seq_lens=pi.seq_lens[k], q_nope128=pi.q_nope128[k], q_pe_raw=pi.q_pe_raw[k],
                             c_kv_raw=pi.c_kv_raw[k], k_pe_raw=pi.k_pe_raw[k])
    rows = check_prolog_outputs(ok, qa[k], qp[k], table=table, what="10-token request")
    check_rows_bf16(c_after, x.cache, ok, bt[k], rows, "10-token request rows", table=table)  # and nothing else changed


def test_up_project_small(dev):
    rng = np.random.default_rng(19)
    for B, q, H in ((1, 1, 1), (37, 1, 16), (5, 4, 128), (3, 8, 3), (9, 8, 16), (100, 1, 4)):  # M = 1 .. 100
        pi = make_prolog_inputs(B, q, H, [q] * B, seed=20)
        a = (rng.standard_normal((B, q, H, 512)) * 0.5).astype(np.float32)
        o = mla.mla_up_project(torch.from_numpy(a).to(dev), bf16_dev(pi.w_uv, dev))
        torch.cuda.synchronize()
        w = bf16_bits_to_f64(pi.w_uv)
        exact = up_project_ref(a.astype(np.float64), w)
        terms = up_project_ref(np.abs(a.astype(np.float64)), np.abs(w))
        check_bf16(bits_of(o), exact, terms, 2.0**-8, f"up-projection B{B} q{q} H{H}")
        got = bf16_bits_to_f64(bits_of(o))
        rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
        assert rel <= 5e-3, f"up-projection rel-L2 {rel}"


def check_o_project(o_bits, w_o_bits, y_bits, what):
    """y against the oracle's output projection of the same bf16 inputs."""
    o = bf16_bits_to_f64(o_bits)
    w = bf16_bits_to_f64(w_o_bits)
    exact = o_project_ref(o, w)
    terms = o_project_ref(np.abs(o), np.abs(w))
    K = w.shape[1]
    check_bf16(y_bits, exact, terms, K * 2.0**-24, what)
    got = bf16_bits_to_f64(y_bits)
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    assert rel <= 5e-3, f"{what}: rel-L2 {rel}"


O_PROJ = [
    # (batch, q_len, heads, n_out): K = 128 heads -> slices of 256 columns
    (1, 1, 2, 64),  # K 256: one chunk, one slice
    (3, 2, 4, 128),  # K 512: two slices
    (37, 1, 16, 192),  # K 2048: eight slices; 37 rows (a ragged 16-row block)
    (9, 8, 8, 64),  # 72 rows: 128-row chunks, four slices
    (130, 1, 2, 64),  # 130 rows: two 128-row chunks
    (5, 1, 6, 320),  # K 768: six chunks, two slices; 320 outputs: 64 per workgroup
    (2, 1, 4, 256),  # 128 outputs per workgroup
    (40, 1, 2, 384),  # 40 rows (64-row chunks), 128 outputs per workgroup
]


@pytest.mark.parametrize("case", O_PROJ, ids=lambda c: f"B{c[0]}q{c[1]}H{c[2]}N{c[3]}")
def test_o_project_small(dev, case):
    B, q, H, N = case
    rng = np.random.default_rng(31)
    o = to_bf16_bits(rng.standard_normal((B, q, H, 128)).astype(np.float32))
    w = to_bf16_bits((rng.standard_normal((N, H * 128)) / np.sqrt(H * 128)).astype(np.float32))
    y = mla.mla_o_project(bf16_dev(o, dev), bf16_dev(w, dev))
    torch.cuda.synchronize()
    check_o_project(o, w, bits_of(y), f"o-projection B{B} q{q} H{H} N{N}")


@pytest.mark.parametrize("name", ["dsv3", "mtp8"])
def test_o_project_full_size(dev, name):
    """7168 x 16384 weights at 32 and 128 query rows."""
    x = make_config(name)
    pi = make_prolog_inputs(x.batch, x.q_len, x.heads, x.seq_lens, seed=CONFIGS[name]["seed"] + 300, hidden=7168)
    o = to_bf16_bits(np.random.default_rng(32).standard_normal((x.batch, x.q_len, x.heads, 128)).astype(np.float32))
    y = mla.mla_o_project(bf16_dev(o, dev), bf16_dev(pi.w_o, dev))
    torch.cuda.synchronize()
    check_o_project(o, pi.w_o, bits_of(y), f"{name} o-projection")


# ---- the chain: prolog -> decode -> up-projection against the oracle's chain ---------------


def _chain(dev, x, pi, fp8, idx=None):
    """GPU chain and the oracle's; returns the comparisons' inputs."""
    if fp8:
        qa, qp, codes, exps = run_prolog(pi, x.cache_codes, x.cache_exps, x.block_table, dev)
        plan = mla.binding.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page)
        out, lse = mla.binding.mla_decode_fp8(
            plan, bf16_dev(qa, dev), bf16_dev(qp, dev), torch.from_numpy(codes).to(dev), torch.from_numpy(exps).to(dev),
            torch.from_numpy(x.block_table).to(dev), torch.from_numpy(x.seq_lens).to(dev), x.softmax_scale,
        )
    else:
        qa, qp, cache, _ = run_prolog(pi, x.cache, None, x.block_table, dev)
        plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page)
        out, lse = mla.mla_decode(
            plan, bf16_dev(qa, dev), bf16_dev(qp, dev), bf16_dev(cache, dev), torch.from_numpy(x.block_table).to(dev),
            torch.from_numpy(x.seq_lens).to(dev), x.softmax_scale,
        )
    o = mla.mla_up_project(out, bf16_dev(pi.w_uv, dev))
    y = None if pi.w_o is None else mla.mla_o_project(o, bf16_dev(pi.w_o, dev))
    torch.cuda.synchronize()
    y = None if y is None else bf16_bits_to_f64(bits_of(y))
    out, lse, o = out.cpu().double().numpy(), lse.cpu().double().numpy(), bf16_bits_to_f64(bits_of(o))
    # the oracle's chain: its prolog, its rows appended, its decode on the
    # bf16 queries the decode entry takes, its up-projection
    q_abs, q_pe, rows = oracle_prolog(pi)
    q16 = to_bf16_bits(bf16_round(q_abs).astype(np.float32))
    p16 = to_bf16_bits(bf16_round(q_pe).astype(np.float32))
    if fp8:
        q = [quantize_row_fp8(r) for r in rows.reshape(-1, 576)]
        codes = append_ref(x.cache_codes, x.block_table, x.seq_lens, np.stack([c for c, _ in q]).reshape(rows.shape))
        exps = append_ref(x.cache_exps, x.block_table, x.seq_lens, np.array([e for _, e in q], np.uint8).reshape(rows.shape[:2]))
        xo = dataclasses.replace(x, q_nope=q16, q_pe=p16, cache_codes=codes.astype(np.uint8), cache_exps=exps.astype(np.uint8))
        ref_o, ref_l, rms, s_abs = t8.oracle(xo, idx)
    else:
        cache = append_ref(x.cache_f64(), x.block_table, x.seq_lens, rows)
        xo = dataclasses.replace(x, q_nope=q16, q_pe=p16, cache=to_bf16_bits(cache.astype(np.float32)))
        ref_o, ref_l = t16.oracle(xo, idx)
        rms = s_abs = None
    sel = slice(None) if idx is None else np.asarray(idx)
    w = bf16_bits_to_f64(pi.w_uv)
    ref_up = up_project_ref(ref_o, w)
    ys = None if y is None else (y[sel], o_project_ref(ref_up, bf16_bits_to_f64(pi.w_o)))
    return out[sel], lse[sel], o[sel], ref_o, ref_l, rms, s_abs, ref_up, ys


def _check_chain(res, fp8, what):
    out, lse, o, ref_o, ref_l, rms, s_abs, ref_up, ys = res
    if fp8:
        t8.compare(out, lse, ref_o, ref_l, rms, s_abs, what)
    else:
        t16.compare(out, lse, ref_o, ref_l, what)
    rel = float(np.linalg.norm(o - ref_up) / np.linalg.norm(ref_up))
    rel_out = float(np.linalg.norm(out - ref_o) / np.linalg.norm(ref_o))
    print(f"{what} up-projected: max-abs {np.max(np.abs(o - ref_up)):.3e} rel-L2 {rel:.3e}", flush=True)
    # W_UV (random, 128 x 512 per head) keeps a relative error's size within a
    # factor ~1 for errors not aligned with its rows; the bf16 roundings of the
    # up-projection add about 2^-9
    assert rel <= 2 * rel_out + 5e-3, f"{what}: up-projected rel-L2 {rel} (attention output's {rel_out})"
    if ys is not None:
        y, ref_y = ys
        rel_y = float(np.linalg.norm(y - ref_y) / np.linalg.norm(ref_y))
        print(f"{what} output projection: rel-L2 {rel_y:.3e}", flush=True)
        # W_O (random, 7168 x 16384) mixes all heads: the error's relative
        # size carries over as for W_UV, plus the output's own bf16 rounding
        assert rel_y <= 2 * rel + 5e-3, f"{what}: output projection rel-L2 {rel_y} (up-projected {rel})"


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_chain_small(dev, fp8):
    B, H, q, page, lens = 4, 16, 2, 16, [2, 30, 77, 140]
    x = (make_inputs_fp8 if fp8 else make_inputs)(B, H, q, page, lens, seed=21)
    pi = make_prolog_inputs(B, q, H, x.seq_lens, seed=22, hidden=256)
    _check_chain(_chain(dev, x, pi, fp8), fp8, f"chain {'fp8' if fp8 else 'bf16'}")


# ---- full size: the 128-head workloads, sampled requests for the decode ---------------------


@pytest.mark.parametrize("name", ["dsv3", "mtp8"])
def test_prolog_full_size(dev, name):
    x = make_config(name)
    c = CONFIGS[name]
    pi = make_prolog_inputs(x.batch, x.q_len, x.heads, x.seq_lens, seed=c["seed"] + 100)
    qa, qp, c_after, _ = run_prolog(pi, x.cache, None, x.block_table, dev)
    rows = check_prolog_outputs(pi, qa, qp, what=f"{name}")
    check_rows_bf16(c_after, x.cache, pi, x.block_table, rows, f"{name} rows")
    a = (np.random.default_rng(23).standard_normal((x.batch, x.q_len, x.heads, 512)) * 0.5).astype(np.float32)
    o = mla.mla_up_project(torch.from_numpy(a).to(dev), bf16_dev(pi.w_uv, dev))
    torch.cuda.synchronize()
    w = bf16_bits_to_f64(pi.w_uv)
    check_bf16(bits_of(o), up_project_ref(a.astype(np.float64), w),
               up_project_ref(np.abs(a.astype(np.float64)), np.abs(w)), 2.0**-8, f"{name} up-projection")


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_chain_dsv3_sampled(dev, fp8):
    """The whole chain at 32 requests x 4096 tokens x 128 heads; the oracle's
    decode on 3 sampled requests."""
    c = CONFIGS["dsv3"]
    x = make_config_fp8("dsv3") if fp8 else make_config("dsv3")
    pi = make_prolog_inputs(x.batch, x.q_len, x.heads, x.seq_lens, seed=c["seed"] + 200, hidden=7168)
    _check_chain(_chain(dev, x, pi, fp8, idx=[0, 13, 31]), fp8, f"dsv3 chain {'fp8' if fp8 else 'bf16'}")
