"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch each one.  A pin set that a dropped term, a wrong sign or index
or a transposed operand slips through would not be a pin."""
import math

import numpy as np
import pytest

from oracle.mla_oracle import gather_kv_rows, visible_keys
from tests import oracle_pins


def _make(score_fn=None, rows_fn=None, n_fn=None, v_slice=slice(0, 512), lse_fn=None, normalize=True, q_fn=None):
    score_fn = score_fn or (lambda q, K, scale: scale * (q @ K.T))
    rows_fn = rows_fn or gather_kv_rows
    n_fn = n_fn or visible_keys
    lse_fn = lse_fn or (lambda m, z: m + np.log(z))
    q_fn = q_fn or (lambda qn, qp, b, j: np.concatenate([qn[b, j], qp[b, j]], axis=-1))

    def ref(q_nope, q_pe, cache, block_table, seq_lens, scale):
        B, q_len, H, _ = q_nope.shape
        out = np.zeros((B, q_len, H, 512))
        lse = np.zeros((B, q_len, H))
        for b in range(B):
            L = int(seq_lens[b])
            K_all = rows_fn(cache, block_table[b], 0, L)
            for j in range(q_len):
                n = max(0, min(L, n_fn(L, q_len, j)))
                q = q_fn(q_nope, q_pe, b, j)
                K = K_all[:n]
                if n == 0:
                    out[b, j] = np.nan
                    lse[b, j] = np.nan
                    continue
                s = score_fn(q, K, scale)
                m = s.max(axis=-1, keepdims=True)
                z = np.exp(s - m).sum(axis=-1, keepdims=True)
                ls = lse_fn(m, z)
                w = np.exp(s - ls) if normalize else np.exp(s - m)
                out[b, j] = w @ K[:, v_slice]
                lse[b, j] = ls[..., 0]
        return out, lse

    return ref


def _swap_page_slot(cache, bt_row, lo, hi):
    P = cache.shape[1]
    t = np.arange(lo, hi)
    # page and slot indices exchanged (clamped so the access stays in range)
    return cache[np.asarray(bt_row)[np.minimum(t % P, len(bt_row) - 1)] % cache.shape[0], np.minimum(t // P, P - 1), :]


MUTANTS = {
    "dropped_rope_term": _make(q_fn=lambda qn, qp, b, j: np.concatenate([qn[b, j], 0 * qp[b, j]], axis=-1)),
    "score_sign": _make(score_fn=lambda q, K, scale: -scale * (q @ K.T)),
    "scale_sqrt576": _make(score_fn=lambda q, K, scale: (q @ K.T) / math.sqrt(576.0)),
    "mask_off_by_one": _make(n_fn=lambda L, q_len, j: L - q_len + j),
    "mask_query_swapped": _make(n_fn=lambda L, q_len, j: L - j),
    "v_wrong_slice": _make(v_slice=slice(64, 576)),
    "page_slot_swapped": _make(rows_fn=_swap_page_slot),
    "lse_log2": _make(lse_fn=lambda m, z: (m + np.log(z)) / math.log(2.0)),
    "unnormalized_out": _make(normalize=False),
    "head_index_shift": _make(q_fn=lambda qn, qp, b, j: np.concatenate([qn[b, j], np.roll(qp[b, j], 1, axis=0)], axis=-1)),
    "query_index_swapped": _make(q_fn=lambda qn, qp, b, j: np.concatenate([qn[b, qn.shape[1] - 1 - j], qp[b, qn.shape[1] - 1 - j]], axis=-1)),
    "q_transposed_dims": _make(q_fn=lambda qn, qp, b, j: np.concatenate([qn[b, j][:, ::-1], qp[b, j]], axis=-1)),
}

# pins other than brute force: each mutant must also be caught by a structural pin
STRUCTURAL = [p for p in oracle_pins.ALL_PINS if p is not oracle_pins.pin_brute_force]


def _caught(ref, pins):
    hits = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(ref)
        except (AssertionError, IndexError, ValueError):
            hits.append(pin.__name__)
    return hits


def test_unmutated_copy_passes_all_pins():
    assert _caught(_make(), oracle_pins.ALL_PINS) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ref = MUTANTS[name]
    assert _caught(ref, [oracle_pins.pin_brute_force]), f"{name} passes brute force"
    hits = _caught(ref, STRUCTURAL)
    assert hits, f"{name} passes every structural pin"
