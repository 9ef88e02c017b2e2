"""Plant plausible mistakes in copies of the prolog/epilog oracle (on the CPU)
and check that at least one pin catches each: a wrong sign, a wrong pairing,
a dropped term, an off-by-one position or exponent, a transposed operand."""
import types

import numpy as np
import pytest

from oracle import mla_prolog_oracle as mo
from tests.test_oracle_prolog import ORACLE, PINS


def _rope_sign(x, cos, sin):
    x = np.asarray(x, np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * cos + b * sin  # the rotation's sine with the wrong sign
    out[..., 1::2] = -a * sin + b * cos
    return out


def _rope_half_split(x, cos, sin):
    x = np.asarray(x, np.float64)
    a, b = x[..., :32], x[..., 32:]  # pairs (x[i], x[i + 32]) instead of (x[2i], x[2i + 1])
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def _rms_no_eps(x, w, eps):
    return mo.rmsnorm_ref(x, w, 0.0)


def _rms_sum(x, w, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps) * np.asarray(w, np.float64)


def _positions_plus_one(seq_lens, q_len):
    return mo.positions(seq_lens, q_len) + 1


def _append_swapped(cache, block_table, seq_lens, rows):
    out = np.array(cache, copy=True)
    P = cache.shape[1]
    pos = mo.positions(seq_lens, rows.shape[1])
    for b in range(rows.shape[0]):
        for j in range(rows.shape[1]):
            t = int(pos[b, j])
            out[int(block_table[b, min(t % P, block_table.shape[1] - 1)]) % cache.shape[0], min(t // P, P - 1)] = rows[b, j]
    return out


def _quantize_exp_plus_one(row):
    row = np.asarray(row, np.float64)
    _, e = mo.quantize_row_fp8(row)
    e += 1  # one exponent too coarse: still in range, but not the smallest
    codes = mo.e4m3_round(np.ldexp(row, -(e - 127)))
    return codes, e


def _o_project_dim_major(o, W_O):
    o = np.asarray(o, np.float64)
    x = np.swapaxes(o, -1, -2).reshape(o.shape[:-2] + (-1,))  # dims outer, heads inner
    return x @ np.asarray(W_O, np.float64).T


def _up_project_transposed_heads(out, W_UV):
    return np.einsum("...hc,hdc->...hd", np.asarray(out, np.float64), np.asarray(W_UV, np.float64)[::-1])


def _prolog_no_norm_weight(q_nope128, q_pe_raw, W_UK, c_kv_raw, kv_norm_w, rms_eps, k_pe_raw, rope_cos, rope_sin, seq_lens):
    return mo.prolog_ref(q_nope128, q_pe_raw, W_UK, c_kv_raw, np.ones_like(kv_norm_w), rms_eps, k_pe_raw, rope_cos,
                         rope_sin, seq_lens)


def _prolog_absorb_transposed(q_nope128, q_pe_raw, W_UK, c_kv_raw, kv_norm_w, rms_eps, k_pe_raw, rope_cos, rope_sin, seq_lens):
    q_abs, q_pe, rows = mo.prolog_ref(q_nope128, q_pe_raw, W_UK, c_kv_raw, kv_norm_w, rms_eps, k_pe_raw, rope_cos,
                                      rope_sin, seq_lens)
    # the right shape from the wrong contraction: rows and heads of W_UK mixed up
    return mo.absorb_query(np.asarray(q_nope128), np.asarray(W_UK)[::-1]), q_pe, rows


MUTANTS = {
    "rope_sign": dict(rope_ref=_rope_sign),
    "rope_half_split_pairs": dict(rope_ref=_rope_half_split),
    "rmsnorm_without_eps": dict(rmsnorm_ref=_rms_no_eps),
    "rmsnorm_sum_not_mean": dict(rmsnorm_ref=_rms_sum),
    "positions_off_by_one": dict(positions=_positions_plus_one),
    "append_page_slot_swapped": dict(append_ref=_append_swapped),
    "row_exponent_off_by_one": dict(quantize_row_fp8=_quantize_exp_plus_one),
    "o_project_dim_major_concat": dict(o_project_ref=_o_project_dim_major),
    "up_project_heads_mixed": dict(up_project_ref=_up_project_transposed_heads),
    "prolog_drops_norm_weight": dict(prolog_ref=_prolog_no_norm_weight),
    "prolog_absorbs_wrong_head": dict(prolog_ref=_prolog_absorb_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_the_mutant(name):
    impl = types.SimpleNamespace(**vars(ORACLE))
    for k, fn in MUTANTS[name].items():
        setattr(impl, k, fn)
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except Exception as e:  # an assertion, or a shape error the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches {name}"


def test_pins_pass_on_the_oracle_itself():
    for pin in PINS:
        pin(ORACLE)
