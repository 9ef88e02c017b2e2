"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes a reference function with the signature of
``oracle.mla_decode_ref`` and raises AssertionError when it disagrees with
what the mathematics fixes (brute force, closed forms, scipy's softmax, the
unabsorbed multi-head form, invariances).  The same pins are run against
deliberately broken copies of the reference in test_oracle_mutants.py, to show
that a plausible mistake anywhere in it is caught.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special

from oracle import brute_force_ref, mha_unabsorbed_ref, mla_decode_split_ref
from workloads import make_inputs

SCALE = 1.0 / math.sqrt(192.0)


def _tiny(seed=11, batch=2, heads=3, q_len=1, page=4, lens=(6, 11)):
    x = make_inputs(batch, heads, q_len, page, list(lens), seed)
    return x, x.q_nope_f64(), x.q_pe_f64(), x.cache_f64()


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def pin_brute_force(ref):
    """Pure-Python loops (math module only) on tiny inputs, q_len 1 and 2."""
    for q_len, lens in ((1, (6, 11)), (2, (5, 9))):
        x, qn, qp, c = _tiny(seed=21 + q_len, q_len=q_len, lens=lens)
        out, lse = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
        bo, bl = brute_force_ref(qn.tolist(), qp.tolist(), c.tolist(), x.block_table.tolist(), x.seq_lens.tolist(), SCALE)
        _close(out, bo, 1e-12, "brute force out")
        _close(lse, bl, 1e-12, "brute force lse")


def pin_textbook_scipy(ref):
    """Dense contiguous layout (identity block table) against scipy softmax/logsumexp."""
    rng = np.random.default_rng(5)
    P, L, H = 8, 29, 4
    npg = -(-L // P)
    dense = rng.standard_normal((npg * P, 576))
    cache = dense.reshape(npg, P, 576)
    bt = np.arange(npg, dtype=np.int32)[None, :]
    qn = rng.standard_normal((1, 1, H, 512))
    qp = rng.standard_normal((1, 1, H, 64))
    out, lse = ref(qn, qp, cache, bt, [L], SCALE)
    q = np.concatenate([qn[0, 0], qp[0, 0]], axis=1)
    s = SCALE * (q @ dense[:L].T)
    _close(out[0, 0], scipy.special.softmax(s, axis=1) @ dense[:L, :512], 1e-12, "scipy out")
    _close(lse[0, 0], scipy.special.logsumexp(s, axis=1), 1e-12, "scipy lse")


def pin_single_token(ref):
    """One visible key: out is that key's c_kv, lse is its scaled score."""
    rng = np.random.default_rng(6)
    P, H = 16, 5
    cache = rng.standard_normal((3, P, 576))
    bt = np.array([[2, 0]], dtype=np.int32)
    qn = rng.standard_normal((1, 1, H, 512))
    qp = rng.standard_normal((1, 1, H, 64))
    out, lse = ref(qn, qp, cache, bt, [1], SCALE)
    row = cache[2, 0]
    for h in range(H):
        s = SCALE * (sum(qn[0, 0, h, d] * row[d] for d in range(512)) + sum(qp[0, 0, h, d] * row[512 + d] for d in range(64)))
        assert abs(lse[0, 0, h] - s) < 1e-12, "single-token lse"
        _close(out[0, 0, h], row[:512], 1e-15, "single-token out")
    # the draft query 0 of an MTP pair with L = 2 also sees exactly one key
    qn2 = rng.standard_normal((1, 2, H, 512))
    qp2 = rng.standard_normal((1, 2, H, 64))
    out2, _ = ref(qn2, qp2, cache, bt, [2], SCALE)
    for h in range(H):
        _close(out2[0, 0, h], row[:512], 1e-15, "MTP query-0 single key")


def pin_zero_query(ref):
    """q = 0: uniform weights, out = mean of V rows, lse = ln(n)."""
    x, qn, qp, c = _tiny(seed=7, lens=(13, 4))
    qn[:] = 0.0
    qp[:] = 0.0
    out, lse = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        rows = np.array([c[x.block_table[b, t // x.page], t % x.page, :512] for t in range(L)])
        for h in range(x.heads):
            _close(out[b, 0, h], rows.mean(axis=0), 1e-13, "zero-query out")
            assert abs(lse[b, 0, h] - math.log(L)) < 1e-13, "zero-query lse"


def pin_identical_keys(ref):
    """Every key the same row r: out = r[:512], lse = s(r) + ln(n)."""
    rng = np.random.default_rng(8)
    P, H, L = 4, 3, 10
    r = rng.standard_normal(576)
    cache = np.broadcast_to(r, (3, P, 576)).copy()
    bt = np.array([[1, 2, 0]], dtype=np.int32)
    qn = rng.standard_normal((1, 1, H, 512))
    qp = rng.standard_normal((1, 1, H, 64))
    out, lse = ref(qn, qp, cache, bt, [L], SCALE)
    for h in range(H):
        s = SCALE * float(np.dot(np.concatenate([qn[0, 0, h], qp[0, 0, h]]), r))
        assert abs(lse[0, 0, h] - (s + math.log(L))) < 1e-12, "identical-keys lse"
        _close(out[0, 0, h], r[:512], 1e-13, "identical-keys out")


def pin_rope_shift(ref):
    """All keys share k_pe = u: adding delta to q_pe shifts every score by
    scale*(delta.u), so out is unchanged and lse moves by that amount."""
    x, qn, qp, c = _tiny(seed=9, lens=(7, 12))
    rng = np.random.default_rng(10)
    u = rng.standard_normal(64)
    c[:, :, 512:] = u
    delta = rng.standard_normal(qp.shape)
    o1, l1 = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
    o2, l2 = ref(qn, qp + delta, c, x.block_table, x.seq_lens, SCALE)
    _close(o2, o1, 1e-12, "rope shift out")
    _close(l2 - l1, SCALE * (delta @ u), 1e-12, "rope shift lse")


def pin_two_tokens(ref):
    """Two keys with hand-set scores: weights are the logistic of the score gap."""
    H = 1
    cache = np.zeros((1, 2, 576))
    # scores: s0 = SCALE * 3 (from the latent part), s1 = SCALE * (-2) (from the rope part)
    cache[0, 0, 0] = 3.0
    cache[0, 1, 512] = -2.0
    cache[0, 0, 1] = 10.0  # V rows differ in column 1 and 2
    cache[0, 1, 2] = 20.0
    qn = np.zeros((1, 1, H, 512))
    qp = np.zeros((1, 1, H, 64))
    qn[0, 0, 0, 0] = 1.0
    qp[0, 0, 0, 0] = 1.0
    bt = np.array([[0]], dtype=np.int32)
    out, lse = ref(qn, qp, cache, bt, [2], SCALE)
    s0, s1 = 3.0 * SCALE, -2.0 * SCALE
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 - w0
    expect = np.zeros(512)
    expect[0] = w0 * 3.0
    expect[1] = w0 * 10.0
    expect[2] = w1 * 20.0
    _close(out[0, 0, 0], expect, 1e-13, "two-token out")
    assert abs(lse[0, 0, 0] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-13, "two-token lse"


def pin_unabsorbed(ref):
    """Absorbed form against standard MHA on the decompressed cache (192-d QK, 128-d V)."""
    from oracle import absorb_query

    rng = np.random.default_rng(12)
    for q_len, lens in ((1, (9, 17)), (2, (6, 10))):
        x, _, qp, c = _tiny(seed=13 + q_len, q_len=q_len, lens=lens)
        H = x.heads
        W_UK = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
        W_UV = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
        qn128 = rng.standard_normal((x.batch, q_len, H, 128))
        out, lse = ref(absorb_query(qn128, W_UK), qp, c, x.block_table, x.seq_lens, SCALE)
        o_mha, l_mha = mha_unabsorbed_ref(qn128, qp, c, x.block_table, x.seq_lens, W_UK, W_UV, SCALE)
        o_abs = np.einsum("bjhc,hdc->bjhd", out, W_UV)
        _close(o_abs, o_mha, 1e-11, "unabsorbed out")
        _close(lse, l_mha, 1e-11, "unabsorbed lse")


def pin_page_permutation(ref):
    """Moving pages to new physical slots (and fixing the block table) changes nothing;
    the identity block table equals a dense contiguous computation."""
    x, qn, qp, c = _tiny(seed=14, lens=(9, 15))
    o1, l1 = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
    rng = np.random.default_rng(15)
    perm = rng.permutation(c.shape[0])  # new slot of old page p is perm[p]
    c2 = np.empty_like(c)
    c2[perm] = c
    bt2 = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1)
    o2, l2 = ref(qn, qp, c2, bt2, x.seq_lens, SCALE)
    _close(o2, o1, 0.0, "page permutation out")
    _close(l2, l1, 0.0, "page permutation lse")
    # dense contiguous layout for request 0 (its pages in order, one per slot)
    L = int(x.seq_lens[0])
    npg = -(-L // x.page)
    c3 = c[x.block_table[0, :npg]]
    bt3 = np.arange(npg, dtype=np.int32)[None, :]
    o3, l3 = ref(qn[:1], qp[:1], c3, bt3, x.seq_lens[:1], SCALE)
    _close(o3, o1[:1], 0.0, "dense layout out")
    _close(l3, l1[:1], 0.0, "dense layout lse")


def pin_split_merge(ref):
    """Any partition of the key range merges (log-sum-exp) to the unsplit result."""
    for q_len in (1, 2):
        x, qn, qp, c = _tiny(seed=16 + q_len, q_len=q_len, lens=(23, 40))
        o, l = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
        rng = np.random.default_rng(17)
        plans = [
            [[], []],
            [[1], [39]],
            [[8, 16], [4, 8, 12, 16, 20, 24, 28, 32, 36]],
            [list(range(1, 23)), list(range(1, 40))],
            [sorted(rng.choice(np.arange(1, 23), 5, replace=False).tolist()), sorted(rng.choice(np.arange(1, 40), 7, replace=False).tolist())],
        ]
        for cuts in plans:
            os_, ls_ = mla_decode_split_ref(qn, qp, c, x.block_table, x.seq_lens, SCALE, cuts)
            _close(os_, o, 1e-12, f"split {cuts} out")
            _close(ls_, l, 1e-12, f"split {cuts} lse")


def pin_mtp_mask(ref):
    """q_len = 2: query 0 equals a q_len = 1 run with L - 1 keys, query 1 one with L."""
    x, qn, qp, c = _tiny(seed=18, q_len=2, lens=(9, 14))
    o, l = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
    o0, l0 = ref(qn[:, :1], qp[:, :1], c, x.block_table, x.seq_lens - 1, SCALE)
    o1, l1 = ref(qn[:, 1:], qp[:, 1:], c, x.block_table, x.seq_lens, SCALE)
    _close(o[:, :1], o0, 1e-13, "mtp query 0 out")
    _close(l[:, :1], l0, 1e-13, "mtp query 0 lse")
    _close(o[:, 1:], o1, 1e-13, "mtp query 1 out")
    _close(l[:, 1:], l1, 1e-13, "mtp query 1 lse")


def pin_batch_order(ref):
    """Reordering the requests reorders the outputs and nothing else."""
    x, qn, qp, c = _tiny(seed=19, batch=3, lens=(5, 12, 8))
    o, l = ref(qn, qp, c, x.block_table, x.seq_lens, SCALE)
    p = np.array([2, 0, 1])
    o2, l2 = ref(qn[p], qp[p], c, x.block_table[p], x.seq_lens[p], SCALE)
    _close(o2, o[p], 0.0, "batch order out")
    _close(l2, l[p], 0.0, "batch order lse")


ALL_PINS = [
    pin_brute_force,
    pin_textbook_scipy,
    pin_single_token,
    pin_zero_query,
    pin_identical_keys,
    pin_rope_shift,
    pin_two_tokens,
    pin_unabsorbed,
    pin_page_permutation,
    pin_split_merge,
    pin_mtp_mask,
    pin_batch_order,
]
