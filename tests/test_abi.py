"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import decode_attention_absorbed_amd as mla
from decode_attention_absorbed_amd import binding as bnd

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mla_decode.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_\w+)\s*\(", src)))


def test_header_declares_exactly_the_exported_symbols():
    assert declared_functions() == sorted(bnd.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = mla.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = mla.lib()
    for code, name in [(0, "MLA_OK"), (1, "MLA_ERR_INVALID_ARGUMENT"), (2, "MLA_ERR_UNSUPPORTED"),
                       (3, "MLA_ERR_WORKSPACE_TOO_SMALL"), (4, "MLA_ERR_HIP"), (5, "MLA_ERR_OUT_OF_MEMORY")]:
        assert L.mla_status_string(code).decode() == name


@pytest.mark.parametrize(
    "args,status",
    [
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=16, num_cus=8), 0),
        (dict(seq_lens=[], q_len=1, num_heads=16, page_size=16, num_cus=8), 1),
        (dict(seq_lens=[5], q_len=0, num_heads=16, page_size=16, num_cus=8), 1),
        (dict(seq_lens=[5], q_len=9, num_heads=16, page_size=16, num_cus=8), 2),
        (dict(seq_lens=[5], q_len=1, num_heads=0, page_size=16, num_cus=8), 1),
        (dict(seq_lens=[5], q_len=1, num_heads=129, page_size=16, num_cus=8), 2),
        (dict(seq_lens=[9], q_len=8, num_heads=128, page_size=16, num_cus=8), 0),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=8, num_cus=8), 2),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=48, num_cus=8), 2),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=8192, num_cus=8), 2),
        (dict(seq_lens=[1], q_len=2, num_heads=16, page_size=16, num_cus=8), 1),
        (dict(seq_lens=[5, 0], q_len=1, num_heads=16, page_size=16, num_cus=8), 1),
        (dict(seq_lens=[(1 << 24) + 1], q_len=1, num_heads=16, page_size=16, num_cus=8), 2),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=16, num_cus=0), 1),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=16, num_cus=65536), 0),
        (dict(seq_lens=[5], q_len=1, num_heads=16, page_size=16, num_cus=65537), 1),
    ],
)
def test_plan_argument_checks(args, status):
    if status == 0:
        p = mla.mla_decode_plan_host(**args)
        assert p.handle
        p.destroy()
    else:
        with pytest.raises(mla.MLAError) as e:
            mla.mla_decode_plan_host(**args)
        assert e.value.status == status
        assert mla.lib().mla_last_error().decode() != ""


def test_plan_out_null_and_query_null():
    L = mla.lib()
    lens = (ctypes.c_int32 * 1)(5)
    assert L.mla_decode_plan_host(lens, 1, 1, 16, 16, 8, None) == 1
    assert L.mla_plan_query(None, 0) == -1
    assert L.mla_decode_workspace_bytes(None) == 0
    assert L.mla_plan_copy(None, None, None) == 1
    L.mla_decode_plan_destroy(None)  # no-op


class _Fake:
    """Non-null, suitably aligned fake device addresses (never dereferenced:
    every check below fails on the host before any HIP call)."""

    base = 1 << 40

    def __init__(self):
        self.n = 0

    def __call__(self, align=256):
        self.n += 1
        return self.base + self.n * (1 << 20)


def _call(plan, **over):
    f = _Fake()
    a = dict(
        q=f(), qp=f(), cache=f(), num_pages=100, bt=f(), bt_stride=64, lens=f(), scale=1 / math.sqrt(192),
        out=f(), lse=f(), ws=f(), ws_bytes=plan.workspace_bytes, stream=None,
    )
    a.update(over)
    return mla.lib().mla_decode(
        plan.handle, a["q"], a["qp"], a["cache"], a["num_pages"], a["bt"], a["bt_stride"], a["lens"], a["scale"],
        a["out"], a["lse"], a["ws"], a["ws_bytes"], a["stream"],
    )


@pytest.fixture(scope="module")
def host_plan():
    # one long request split over 64 slots -> the plan needs a workspace
    p = mla.mla_decode_plan_host([4000, 17], 1, 128, 64, 64)
    assert p.workspace_bytes > 0
    yield p
    p.destroy()


def test_decode_rejects_null_pointers(host_plan):
    for k in ("q", "qp", "cache", "bt", "lens", "out", "lse"):
        assert _call(host_plan, **{k: None}) == 1, k


def test_decode_rejects_misalignment(host_plan):
    for k in ("q", "qp", "cache", "out"):
        assert _call(host_plan, **{k: (1 << 40) + 8}) == 1, k
    assert _call(host_plan, lse=(1 << 40) + 2) == 1
    assert _call(host_plan, ws=(1 << 40) + 128) == 1


def test_decode_rejects_bad_sizes(host_plan):
    assert _call(host_plan, num_pages=0) == 1
    assert _call(host_plan, bt_stride=62) == 1  # ceil(4000 / 64) = 63 pages needed
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert _call(host_plan, scale=s) == 1, s


def test_decode_workspace_checks(host_plan):
    assert _call(host_plan, ws_bytes=host_plan.workspace_bytes - 1) == 3
    assert _call(host_plan, ws=None) == 1


def test_decode_refuses_host_only_plan(host_plan):
    assert _call(host_plan) == 1
    assert "mla_decode_plan_host" in mla.lib().mla_last_error().decode()
    assert _call(host_plan, bt_stride=63) == 1  # exactly enough pages is fine up to the plan check


def test_plan_update_argument_checks(host_plan):
    L = mla.lib()
    lens = np.array([3000, 20], dtype=np.int32)
    ptr = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.mla_decode_plan_update(None, ptr, None) == 1
    assert L.mla_decode_plan_update(host_plan.handle, None, None) == 1
    # a host-only plan has no device schedule to update (refused before any HIP call)
    assert L.mla_decode_plan_update(host_plan.handle, ptr, None) == 1
    assert "_plan_host" in L.mla_last_error().decode()
    with pytest.raises(ValueError):
        host_plan.update([1, 2, 3])  # wrong batch
    # the plan is unchanged
    assert host_plan.query(bnd.MLA_Q_NUM_PARTIALS) > 0


def test_plan_query_keys(host_plan):
    assert host_plan.query(bnd.MLA_Q_ROWS_PER_BLOCK) in (64, 128)
    assert host_plan.query(bnd.MLA_Q_TILE_TOKENS) in (32, 64)
    assert host_plan.query(999) == -1


# ---- the FP8 entry points: the same host-side checks --------------------------------------


def _call8(plan, **over):
    f = _Fake()
    a = dict(
        q=f(), qp=f(), codes=f(), scales=f(), num_pages=100, bt=f(), bt_stride=64, lens=f(),
        scale=1 / math.sqrt(192), out=f(), lse=f(), ws=f(), ws_bytes=plan.workspace_bytes, stream=None,
    )
    a.update(over)
    return mla.lib().mla_decode_fp8(
        plan.handle, a["q"], a["qp"], a["codes"], a["scales"], a["num_pages"], a["bt"], a["bt_stride"], a["lens"],
        a["scale"], a["out"], a["lse"], a["ws"], a["ws_bytes"], a["stream"],
    )


@pytest.fixture(scope="module")
def host_plan8():
    p = bnd.mla_decode_fp8_plan_host([4000, 17], 1, 128, 64, 64)
    assert p.workspace_bytes > 0
    assert p.query(bnd.MLA_Q_TILE_TOKENS) == 64 and p.query(bnd.MLA_Q_ROWS_PER_BLOCK) == 128
    yield p
    p.destroy()


def test_fp8_decode_rejects_null_pointers(host_plan8):
    for k in ("q", "qp", "codes", "scales", "bt", "lens", "out", "lse"):
        assert _call8(host_plan8, **{k: None}) == 1, k


def test_fp8_decode_rejects_misalignment(host_plan8):
    for k in ("q", "qp", "codes", "out"):
        assert _call8(host_plan8, **{k: (1 << 40) + 8}) == 1, k
    assert _call8(host_plan8, scales=(1 << 40) + 2) == 1
    assert _call8(host_plan8, ws=(1 << 40) + 128) == 1


def test_fp8_decode_rejects_bad_sizes(host_plan8):
    assert _call8(host_plan8, num_pages=0) == 1
    assert _call8(host_plan8, bt_stride=62) == 1
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert _call8(host_plan8, scale=s) == 1, s
    assert _call8(host_plan8, ws_bytes=host_plan8.workspace_bytes - 1) == 3


def test_plan_kinds_are_not_interchangeable(host_plan, host_plan8):
    # each decode call refuses the other kind's plan before anything else
    assert _call8(host_plan) == 1
    assert "mla_decode_fp8_plan" in mla.lib().mla_last_error().decode()
    assert _call(host_plan8) == 1
    assert "mla_decode_plan" in mla.lib().mla_last_error().decode()


def test_fp8_plan_covers_every_key_once():
    lens = [2, 63, 64, 65, 4000, 20480]
    p = bnd.mla_decode_fp8_plan_host(lens, 2, 128, 16, 256)
    seg = p.segments()
    for b, L in enumerate(lens):
        pieces = sorted((int(s[1]), int(s[2])) for s in seg if s[0] == b)
        assert pieces[0][0] == 0 and pieces[-1][1] == L
        assert all(pieces[i][1] == pieces[i + 1][0] for i in range(len(pieces) - 1))
        assert all(lo % 64 == 0 for lo, _ in pieces)  # pieces start on 64-key tiles
    p.destroy()


# ---- the prolog / epilog entry points -------------------------------------------------------


def _prolog(**over):
    f = _Fake()
    a = dict(
        B=2, q=1, H=128, qn=f(), qpr=f(), wuk=f(), ckv=f(), nw=f(), eps=1e-6, kpe=f(), cs=f(), max_pos=4096,
        lens=f(), bt=f(), bt_stride=64, num_pages=100, page=64, fmt=bnd.MLA_KV_BF16, cache=f(), scales=None,
        qa=f(), qp=f(), stream=None,
    )
    a.update(over)
    return mla.lib().mla_prolog(
        a["B"], a["q"], a["H"], a["qn"], a["qpr"], a["wuk"], a["ckv"], a["nw"], a["eps"], a["kpe"], a["cs"],
        a["max_pos"], a["lens"], a["bt"], a["bt_stride"], a["num_pages"], a["page"], a["fmt"], a["cache"],
        a["scales"], a["qa"], a["qp"], a["stream"],
    )


def test_prolog_rejects_null_pointers():
    for k in ("qn", "qpr", "wuk", "ckv", "nw", "kpe", "cs", "lens", "bt", "cache", "qa", "qp"):
        assert _prolog(**{k: None}) == 1, k
    assert _prolog(fmt=bnd.MLA_KV_FP8, scales=None) == 1
    assert "kv_scales" in mla.lib().mla_last_error().decode()


def test_prolog_rejects_bad_sizes_and_formats():
    for over in (dict(B=0), dict(q=0), dict(q=9), dict(H=0), dict(H=129), dict(B=(1 << 18) + 1, q=8),
                 dict(page=8), dict(page=48),
                 dict(page=8192), dict(max_pos=0), dict(bt_stride=0), dict(num_pages=0), dict(fmt=2),
                 dict(eps=-1.0), dict(eps=float("nan"))):
        assert _prolog(**over) == 1, over


def test_prolog_rejects_misalignment():
    for k in ("qn", "qpr", "wuk", "cs", "qa", "qp", "cache"):
        assert _prolog(**{k: (1 << 40) + 8}) == 1, k
    for k in ("qpr", "ckv", "nw", "kpe", "qp", "cs", "lens", "bt"):
        assert _prolog(**{k: (1 << 40) + 2}) == 1, k


def test_up_project_argument_checks():
    f = _Fake()
    up = mla.lib().mla_up_project
    assert up(1, 1, 128, None, f(), f(), None) == 1
    assert up(1, 1, 128, f(), None, f(), None) == 1
    assert up(1, 1, 128, f(), f(), None, None) == 1
    assert up(0, 1, 128, f(), f(), f(), None) == 1
    assert up((1 << 18) + 1, 8, 128, f(), f(), f(), None) == 1
    assert up(1, 9, 128, f(), f(), f(), None) == 1
    assert up(1, 1, 129, f(), f(), f(), None) == 1
    assert up(1, 1, 128, (1 << 40) + 8, f(), f(), None) == 1
    assert up(1, 1, 128, f(), (1 << 40) + 8, f(), None) == 1
    assert up(1, 1, 128, f(), f(), (1 << 40) + 4, None) == 1


def test_o_project_argument_checks():
    f = _Fake()
    op, ws = mla.lib().mla_o_project, mla.lib().mla_o_project_workspace_bytes
    need = ws(32, 1, 16384, 7168)
    assert need == 8 * 32 * 7168 * 4  # 8 slices of fp32 partials (128 output rows per workgroup)
    assert ws(64, 2, 16384, 7168) == 4 * 128 * 7168 * 4  # above 64 rows: 4 slices
    assert ws(48, 1, 16384, 7168) == 8 * 48 * 7168 * 4
    assert ws(48, 1, 16384, 7104) == 4 * 48 * 7104 * 4  # 7104 = 111 x 64: 64 output rows, 4 slices
    assert ws(1, 1, 768, 64) == 2 * 1 * 64 * 4  # 64 outputs: 4 slices wanted, 6 chunks of 128 -> 2
    assert ws(1, 1, 768, 128) == 2 * 1 * 128 * 4  # 128 outputs: 8 slices wanted -> 2
    for bad in ((0, 1, 256, 64), (1, 9, 256, 64), (1, 1, 100, 64), (1, 1, 256, 96), (1, 1, 0, 64)):
        assert ws(*bad) == 0, bad
    args = lambda **o: [o.get(k, d) for k, d in (("B", 32), ("q", 1), ("K", 16384), ("N", 7168), ("x", f()), ("w", f()),
                                                  ("y", f()), ("ws", f()), ("wsb", need), ("st", None))]
    for over in (dict(x=None), dict(w=None), dict(y=None), dict(ws=None), dict(B=0), dict(q=9), dict(K=100),
                 dict(K=0), dict(N=96), dict(N=0), dict(B=(1 << 17), N=(1 << 12) * 64),
                 dict(x=(1 << 40) + 8), dict(w=(1 << 40) + 8), dict(ws=(1 << 40) + 8), dict(y=(1 << 40) + 4)):
        assert op(*args(**over)) == 1, over
    assert op(*args(wsb=need - 1)) == 3

