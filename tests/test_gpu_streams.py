"""Streams and HIP graphs on an MI355X, through the C ABI.

- One plan shared by calls on two streams at once, each with its own
  workspace (the sharing the ABI allows): every result is bitwise the
  serial one.
- The decode (both kernels of a step) captured in a HIP graph and replayed
  several times, with eager work and new inputs between the replays: every
  replay is bitwise the eager call on the same inputs.  The decode records no
  memset and no allocation, so a capture holds only its kernels.
"""
import dataclasses

import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from decode_attention_absorbed_amd import binding as bnd  # noqa: E402
from workloads import make_inputs, make_inputs_fp8  # noqa: E402

pytestmark = pytest.mark.gpu

LENS = [3000, 700, 65, 2000]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def inputs(kv, seed):
    """Batches of the same cache, pages and request order (one plan serves all
    of them) with the queries of `seed`: the request order of a batch depends on
    its seed, so only the queries are drawn anew."""
    make = make_inputs if kv == "bf16" else make_inputs_fp8
    x = make(len(LENS), 128, 2, 64, LENS, seed=80)
    if seed != 80:
        q = make(len(LENS), 128, 2, 64, LENS, seed=seed)
        x = dataclasses.replace(x, q_nope=q.q_nope, q_pe=q.q_pe)
    return x


def make_plan(kv, x):
    if kv == "bf16":
        return mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, 0)
    return bnd.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page, 0)


def decode(kv, plan, x, t, **kw):
    if kv == "bf16":
        return mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                              x.softmax_scale, **kw)
    return bnd.mla_decode_fp8(plan, t["q_nope"], t["q_pe"], t["cache_codes"], t["cache_exps"], t["block_table"],
                              t["seq_lens"], x.softmax_scale, **kw)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_one_plan_on_two_streams(dev, kv):
    xs = [inputs(kv, 81), inputs(kv, 82)]  # same lengths, different values
    ts = [x.to_torch(dev) for x in xs]
    plan = make_plan(kv, xs[0])
    need = plan.workspace_bytes
    assert need > 0
    serial = []
    for x, t in zip(xs, ts):
        o, l = decode(kv, plan, x, t)
        torch.cuda.synchronize()
        serial.append((o.clone(), l.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    ws = [torch.empty(need, dtype=torch.uint8, device=dev) for _ in range(2)]
    outs = [[], []]
    torch.cuda.synchronize()
    assert not torch.equal(serial[0][0], serial[1][0])
    for o, l in serial:
        assert torch.isfinite(o).all() and torch.isfinite(l).all()
    for _ in range(4):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                outs[k].append(decode(kv, plan, xs[k], ts[k], workspace=ws[k], stream=streams[k]))
    torch.cuda.synchronize()
    for k in range(2):
        for o, l in outs[k]:
            assert torch.equal(o, serial[k][0]) and torch.equal(l, serial[k][1]), k
    plan.destroy()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_decode_replayed_from_a_hip_graph(dev, kv):
    xs = [inputs(kv, 83), inputs(kv, 84), inputs(kv, 85)]
    ts = [x.to_torch(dev) for x in xs]
    plan = make_plan(kv, xs[0])
    # static buffers the graph reads and writes
    st = {k: v.clone() for k, v in ts[0].items()}
    out = torch.empty((xs[0].batch, xs[0].q_len, xs[0].heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((xs[0].batch, xs[0].q_len, xs[0].heads), dtype=torch.float32, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    decode(kv, plan, xs[0], st, out=out, lse=lse, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        decode(kv, plan, xs[0], st, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 2, 0, 2, 1)):
        for k in st:
            st[k].copy_(ts[i][k])  # new inputs, eager
        ref_o, ref_l = decode(kv, plan, xs[i], ts[i])  # eager call with its own buffers
        torch.cuda.synchronize()
        assert torch.isfinite(ref_o).all() and torch.isfinite(ref_l).all()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} (inputs {i})"
    del g
    plan.destroy()
