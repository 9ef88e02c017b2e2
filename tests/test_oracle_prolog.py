"""Pins for the prolog/epilog part of the oracle (CPU only)."""
import math

import numpy as np
import pytest
import torch

import types

from oracle import absorb_query, mha_unabsorbed_ref, mla_decode_ref
from oracle import mla_prolog_oracle
from oracle.mla_oracle_fp8 import e4m3_decode
from workloads import make_inputs

#: the implementation the pins check (tests/test_oracle_prolog_mutants.py swaps
#: single functions of it for planted mistakes)
ORACLE = types.SimpleNamespace(**{k: getattr(mla_prolog_oracle, k) for k in (
    "append_ref", "bf16_round", "o_project_ref", "positions", "prolog_ref", "quantize_row_fp8", "rmsnorm_ref",
    "rope_ref", "rope_table", "up_project_ref")})

SCALE = 1.0 / math.sqrt(192.0)


def _rot(o, x, p, cos, sin):
    return o.rope_ref(x, cos[p], sin[p])


def pin_rope_closed_forms(o):
    cos, sin = o.rope_table(10000.0, 64)
    x = np.random.default_rng(0).standard_normal(64)
    np.testing.assert_array_equal(_rot(o, x, 0, cos, sin), x)  # position 0: identity
    # pair 0 turns by p radians (theta^0 = 1): a quarter turn at p = pi/2 maps
    # (1, 0) to (0, 1)
    c = np.ones(32)
    s = np.zeros(32)
    c[0], s[0] = math.cos(math.pi / 2), math.sin(math.pi / 2)
    e = np.zeros(64)
    e[0] = 1.0
    np.testing.assert_allclose(o.rope_ref(e, c, s)[:2], [0.0, 1.0], atol=1e-15)
    # rotations keep every pair's length
    y = _rot(o, x, 37, cos, sin)
    np.testing.assert_allclose(np.hypot(y[0::2], y[1::2]), np.hypot(x[0::2], x[1::2]), rtol=1e-14)


def pin_rope_relative_positions(o):
    """<R(p) q, R(p') k> = <q, R(p' - p) k>: scores depend on the offset only."""
    cos, sin = o.rope_table(10000.0, 4096)
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for p, pp in ((0, 5), (100, 1000), (3000, 4095)):
        lhs = _rot(o, q, p, cos, sin) @ _rot(o, k, pp, cos, sin)
        rhs = q @ _rot(o, k, pp - p, cos, sin)
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))
    # and rotations compose: R(a) R(b) = R(a + b)
    np.testing.assert_allclose(_rot(o, _rot(o, k, 300, cos, sin), 400, cos, sin), _rot(o, k, 700, cos, sin), atol=1e-11)


def pin_rmsnorm_closed_forms(o):
    rng = np.random.default_rng(2)
    x = rng.standard_normal(512)
    y = o.rmsnorm_ref(x, np.ones(512), 0.0)
    assert abs(np.sqrt((y * y).mean()) - 1.0) < 1e-14  # unit RMS
    np.testing.assert_allclose(o.rmsnorm_ref(7.5 * x, np.ones(512), 0.0), y, rtol=1e-14)  # scale invariance
    c, eps = 3.0, 0.25
    np.testing.assert_allclose(o.rmsnorm_ref(np.full(512, c), np.ones(512), eps), c / math.sqrt(c * c + eps))
    w = rng.standard_normal(512)
    np.testing.assert_allclose(o.rmsnorm_ref(x, w, 1e-6), o.rmsnorm_ref(x, np.ones(512), 1e-6) * w, rtol=1e-14)


def pin_positions_and_append(o):
    x = make_inputs(3, 2, 2, 16, [5, 17, 32], seed=4)
    pos = o.positions(x.seq_lens, 2)
    assert pos.tolist() == [[int(L) - 2, int(L) - 1] for L in x.seq_lens]
    cache = np.zeros((x.num_pages, 16, 3))
    rows = np.arange(3 * 2 * 3, dtype=np.float64).reshape(3, 2, 3) + 1.0
    out = o.append_ref(cache, x.block_table, x.seq_lens, rows)
    # brute force: every written slot holds its row, nothing else changed
    written = np.zeros((x.num_pages, 16), bool)
    for b in range(3):
        for j in range(2):
            t = int(x.seq_lens[b]) - 2 + j
            pg, sl = int(x.block_table[b][t // 16]), t % 16
            np.testing.assert_array_equal(out[pg, sl], rows[b, j])
            written[pg, sl] = True
    assert np.all(out[~written] == 0)


def pin_bf16_round_matches_torch(o):
    v = np.random.default_rng(3).standard_normal(5000) * 10.0 ** np.random.default_rng(4).integers(-5, 5, 5000)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(o.bf16_round(v), t)


def pin_quantize_row_fp8(o):
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 37.0, 1e4):
        row = rng.standard_normal(576) * scale
        codes, e = o.quantize_row_fp8(row)
        f = e - 127
        amax = np.abs(row).max()
        assert math.ldexp(amax, -f) <= 448 < math.ldexp(amax, -(f - 1))  # smallest such f
        back = np.ldexp(e4m3_decode(codes), f)
        big = np.abs(row) >= math.ldexp(2.0**-6, f)  # normal E4M3 range
        assert np.all(np.abs(back - row)[big] <= 2.0**-4 * np.abs(row)[big])


def pin_prolog_reference_pieces(o):
    rng = np.random.default_rng(6)
    B, q, H = 2, 2, 4
    qn, qp = rng.standard_normal((B, q, H, 128)), rng.standard_normal((B, q, H, 64))
    W = rng.standard_normal((H, 128, 512)) / math.sqrt(128)
    ckv, w, kpe = rng.standard_normal((B, q, 512)), rng.standard_normal(512), rng.standard_normal((B, q, 64))
    cos, sin = o.rope_table(10000.0, 200)
    lens = [17, 150]
    q_abs, q_pe, rows = o.prolog_ref(qn, qp, W, ckv, w, 1e-6, kpe, cos, sin, lens)
    # brute force for one head and token
    b, j, h = 1, 1, 3
    np.testing.assert_allclose(q_abs[b, j, h], sum(qn[b, j, h, d] * W[h, d] for d in range(128)), rtol=1e-12)
    p = lens[b] - q + j
    for i in range(32):
        a, c = qp[b, j, h, 2 * i], qp[b, j, h, 2 * i + 1]
        np.testing.assert_allclose(q_pe[b, j, h, 2 * i : 2 * i + 2], [a * cos[p, i] - c * sin[p, i], a * sin[p, i] + c * cos[p, i]], rtol=1e-12)
    x = ckv[b, j]
    np.testing.assert_allclose(rows[b, j, :512], o.bf16_round(x / math.sqrt((x * x).mean() + 1e-6) * w))
    np.testing.assert_array_equal(rows, o.bf16_round(rows))


def pin_up_projection_completes_the_unabsorbed_attention(o):
    """W_UV applied to the absorbed attention's output is the ordinary
    multi-head attention's output (with W_UK absorbed into the query)."""
    rng = np.random.default_rng(7)
    x = make_inputs(2, 3, 2, 8, [11, 25], seed=8)
    cache = x.cache_f64()
    qn128 = rng.standard_normal((2, 2, 3, 128))
    W_UK = rng.standard_normal((3, 128, 512)) / math.sqrt(512)
    W_UV = rng.standard_normal((3, 128, 512)) / math.sqrt(512)
    o_ref, lse_ref = mha_unabsorbed_ref(qn128, x.q_pe_f64(), cache, x.block_table, x.seq_lens, W_UK, W_UV, SCALE)
    out, lse = mla_decode_ref(absorb_query(qn128, W_UK), x.q_pe_f64(), cache, x.block_table, x.seq_lens, SCALE)
    np.testing.assert_allclose(o.up_project_ref(out, W_UV), o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
    # and per head it is the plain matrix-vector product
    np.testing.assert_allclose(o.up_project_ref(out, W_UV)[1, 0, 2], W_UV[2] @ out[1, 0, 2], rtol=1e-12)


def pin_o_projection_per_head_blocks(o):
    """The output projection of the concatenated heads is the sum over heads of
    each head's 128 columns of W_O applied to that head (brute force), and with
    the up-projection it completes the ordinary multi-head attention."""
    rng = np.random.default_rng(9)
    oh = rng.standard_normal((2, 3, 4, 128))
    W = rng.standard_normal((40, 4 * 128))
    y = o.o_project_ref(oh, W)
    assert y.shape == (2, 3, 40)
    for b, j in ((0, 0), (1, 2)):
        ref = sum(W[:, h * 128:(h + 1) * 128] @ oh[b, j, h] for h in range(4))
        np.testing.assert_allclose(y[b, j], ref, rtol=1e-12, atol=1e-12)
        n = 7
        brute = sum(W[n, h * 128 + d] * oh[b, j, h, d] for h in range(4) for d in range(128))
        assert abs(y[b, j, n] - brute) < 1e-10
    # the whole chain: absorbed attention, up-projection, output projection =
    # the unabsorbed multi-head attention's output projected
    x = make_inputs(2, 3, 1, 8, [11, 25], seed=10)
    qn128 = rng.standard_normal((2, 1, 3, 128))
    W_UK = rng.standard_normal((3, 128, 512)) / math.sqrt(512)
    W_UV = rng.standard_normal((3, 128, 512)) / math.sqrt(512)
    W_O = rng.standard_normal((24, 3 * 128))
    o_ref, _ = mha_unabsorbed_ref(qn128, x.q_pe_f64(), x.cache_f64(), x.block_table, x.seq_lens, W_UK, W_UV, SCALE)
    out, _ = mla_decode_ref(absorb_query(qn128, W_UK), x.q_pe_f64(), x.cache_f64(), x.block_table, x.seq_lens, SCALE)
    np.testing.assert_allclose(o.o_project_ref(o.up_project_ref(out, W_UV), W_O), o.o_project_ref(o_ref, W_O), rtol=1e-9, atol=1e-11)


PINS = [pin_rope_closed_forms, pin_rope_relative_positions, pin_rmsnorm_closed_forms, pin_positions_and_append, pin_bf16_round_matches_torch, pin_quantize_row_fp8, pin_prolog_reference_pieces, pin_up_projection_completes_the_unabsorbed_attention, pin_o_projection_per_head_blocks]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ORACLE)
