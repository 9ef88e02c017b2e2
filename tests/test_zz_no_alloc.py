"""The allocation-free entry point against mla_decode (through the C ABI).

mla_decode_noalloc runs the same kernels as mla_decode with the partials of
split requests in the library's per-GPU scratch instead of a caller
workspace, so its outputs must equal mla_decode's bit for bit.  Two calls in
a row, the second with a smaller input, check that the scratch left by the
first call does not leak into the second.
"""
import ctypes

import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from decode_attention_absorbed_amd import binding as bnd  # noqa: E402
from workloads import make_inputs  # noqa: E402


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _noalloc(plan, t, x, out, lse):
    L = mla.lib()
    stream = torch.cuda.current_stream(out.device)
    bt, sl = t["block_table"], t["seq_lens"]
    st = L.mla_decode_noalloc(plan.handle, t["q_nope"].data_ptr(), t["q_pe"].data_ptr(), t["cache"].data_ptr(),
                              int(t["cache"].shape[0]), bt.data_ptr(), int(bt.shape[1]), sl.data_ptr(),
                              float(x.softmax_scale), out.data_ptr(), lse.data_ptr(), stream.cuda_stream)
    bnd._check(st)


@pytest.mark.gpu
def test_noalloc_matches_mla_decode_on_two_calls():
    dev = _dev()
    cases = [
        # split requests (pieces write partials to the scratch), q_len 2 (two row blocks)
        dict(batch=4, heads=128, q_len=2, page=64, lens=[3000, 700, 65, 2000], seed=21),
        # smaller: fewer pieces, fewer rows
        dict(batch=2, heads=64, q_len=1, page=16, lens=[500, 90], seed=22),
    ]
    for c in cases:
        x = make_inputs(c["batch"], c["heads"], c["q_len"], c["page"], c["lens"], seed=c["seed"])
        print(f"no-alloc case B={x.batch} H={x.heads} q_len={x.q_len} lens={list(x.seq_lens)}", flush=True)
        t = x.to_torch(dev)
        plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, 256)
        assert plan.query(bnd.MLA_Q_NUM_PARTIALS) > 0, "the case must split requests"
        ref_o, ref_l = mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                                      x.softmax_scale)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        _noalloc(plan, t, x, out, lse)
        torch.cuda.synchronize()
        # the same kernels on the same plan: bit-identical to mla_decode
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_noalloc_refuses_plans_beyond_its_scratch():
    # 1024 planned compute units over long requests: > 64 MiB of partials.
    # Refused before any HIP call (the pointers are never dereferenced).
    plan = mla.mla_decode_plan_host([131072] * 8, 1, 128, 64, 1024)
    assert plan.workspace_bytes > 64 << 20
    L = mla.lib()
    fake = ctypes.c_void_p(256)
    st = L.mla_decode_noalloc(plan.handle, fake, fake, fake, 1, fake, 1 << 20, fake, 0.07, fake, fake, None)
    assert st == bnd.MLA_ERR_WORKSPACE_TOO_SMALL
    assert b"scratch" in L.mla_last_error()
