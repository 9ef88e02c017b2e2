"""Split planner properties (host-only plans, CPU)."""
import numpy as np
import pytest

import decode_attention_absorbed_amd as mla
from decode_attention_absorbed_amd import binding as bnd
from workloads import CONFIGS, config_lens


def check_plan(lens, q_len, heads, page, num_cus):
    p = mla.mla_decode_plan_host(lens, q_len, heads, page, num_cus)
    seg = p.segments()
    wg = p.workgroups()
    T = p.query(bnd.MLA_Q_TILE_TOKENS)
    rpb = p.query(bnd.MLA_Q_ROWS_PER_BLOCK)
    nrb = p.query(bnd.MLA_Q_NUM_ROW_BLOCKS)
    assert nrb == -(-q_len * heads // rpb)
    lens = np.asarray(lens)
    # coverage: every key of every request exactly once, tile-aligned starts
    cover = [np.zeros(L, dtype=np.int32) for L in lens]
    for b, k0, k1, part in seg:
        assert 0 <= k0 < k1 <= lens[b] and k0 % T == 0
        cover[b][k0:k1] += 1
    for b in range(len(lens)):
        assert np.all(cover[b] == 1), f"request {b} not covered exactly once"
    # partial ids: -1 for whole requests, distinct ids for split ones
    pieces = np.bincount(seg[:, 0], minlength=len(lens))
    ids = seg[seg[:, 3] >= 0, 3]
    assert len(set(ids.tolist())) == len(ids) == p.query(bnd.MLA_Q_NUM_PARTIALS)
    for b, k0, k1, part in seg:
        assert (part < 0) == (pieces[b] == 1)
    # every segment is run once per row block, by workgroups on one XCD
    runs = {}
    for w, (s0, s1, rb, _) in enumerate(wg):
        for s in range(s0, s1):
            runs.setdefault(s, []).append((rb, w))
    assert sorted(runs) == list(range(len(seg)))
    for s, lst in runs.items():
        assert sorted(r for r, _ in lst) == list(range(nrb))
        assert len({w % 8 for _, w in lst}) == 1
    # the busy workgroups fit on the device at once
    busy = int((wg[:, 1] > wg[:, 0]).sum())
    assert busy <= max(nrb, num_cus * (2 if rpb == 64 else 1))
    # combine workgroups: every row of every split request once, each on the
    # XCD that wrote most of its partials, at most an even share per XCD
    cu = p.combine_units()
    split = np.flatnonzero(pieces > 1)
    assert (len(cu) == 0) == (len(split) == 0)
    if len(split):
        per = 4 if pieces.max() <= 16 else 1
        rows = q_len * heads
        first = {b: int(seg[(seg[:, 0] == b) & (seg[:, 3] >= 0), 3].min()) for b in split}
        seen = np.zeros((len(lens), rows), dtype=np.int32)
        xcd_of, local, total = {}, 0, 0
        for s, lst in runs.items():
            if seg[s, 3] >= 0:
                for rb, w in lst:
                    xcd_of[(int(seg[s, 3]), rb)] = w % 8
        for i, (b, p0, n, r0) in enumerate(cu):
            if n == 0:
                continue
            assert pieces[b] > 1 and n == pieces[b] and p0 == first[b] and r0 % per == 0
            seen[b, r0:min(r0 + per, rows)] += 1
            votes = np.bincount([xcd_of[(p0 + k, r0 // rpb)] for k in range(n)], minlength=8)
            local += int(votes[i % 8] == votes.max())
            total += 1
        p.combine_local = local / total
        assert np.all(seen[split] == 1) and np.all(seen[pieces <= 1] == 0)
        units = sum(-(-rows // per) for _ in split)
        assert len(cu) <= 8 * -(-units // 8)
    # workspace size
    slots = p.query(bnd.MLA_Q_NUM_PARTIALS) * nrb
    expect = 0 if slots == 0 else (-(-slots * rpb * 512 * 2 // 256) * 256 + 2 * (-(-slots * rpb * 4 // 256) * 256))
    assert p.workspace_bytes == expect
    return p, seg, wg, T


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_named_workloads_plan(name):
    c = CONFIGS[name]
    lens = config_lens(name)
    p, seg, wg, T = check_plan(lens, c["q_len"], c["heads"], c["page"], 256)
    # balance: tiles per workgroup close to the mean for the big workloads
    load = np.zeros(len(wg))
    for w, (s0, s1, rb, _) in enumerate(wg):
        for s in range(s0, s1):
            load[w] += -(-(seg[s, 2] - seg[s, 1]) // T)
    used = load[load > 0]
    if name != "tiny":
        assert used.max() <= 1.2 * used.mean() + 6, (used.max(), used.mean())
        assert len(used) >= 200  # nearly every CU busy
    if name in ("dsv3", "long"):
        # each request's pieces sit on one XCD; its combine rows run there too
        assert p.combine_local == 1.0


def test_long_request_is_split_across_the_device():
    p, seg, wg, T = check_plan([131072], 1, 128, 64, 256)
    assert len(seg) >= 200


def test_mixed_lengths_do_not_serialise_on_the_long_requests():
    lens = config_lens("mixed")
    p, seg, wg, T = check_plan(lens, 1, 128, 64, 256)
    long_pieces = np.bincount(seg[:, 0], minlength=len(lens))[lens == 20480]
    assert long_pieces.min() >= 5


@pytest.mark.parametrize("num_cus", [1, 2, 7, 64, 256, 1024])
@pytest.mark.parametrize("q_len,heads,page", [(1, 16, 16), (2, 128, 64), (1, 100, 32), (3, 64, 128)])
def test_random_lengths_plan(num_cus, q_len, heads, page):
    rng = np.random.default_rng(num_cus * 7 + q_len)
    lens = rng.integers(q_len, 3000, size=13)
    check_plan(lens, q_len, heads, page, num_cus)


def test_single_slot_never_splits():
    p, seg, wg, T = check_plan([5000, 70, 1], 1, 128, 64, 1)
    assert (seg[:, 3] == -1).all() and p.workspace_bytes == 0


def test_deterministic():
    lens = config_lens("mtp")
    a = mla.mla_decode_plan_host(lens, 2, 128, 64, 256)
    b = mla.mla_decode_plan_host(lens, 2, 128, 64, 256)
    np.testing.assert_array_equal(a.segments(), b.segments())
    np.testing.assert_array_equal(a.workgroups(), b.workgroups())
