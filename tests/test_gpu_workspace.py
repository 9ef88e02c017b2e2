"""Caller-provided buffers on an MI355X: the decode's results do not depend on
what the workspace, out and lse held before the call (every partial the
combine reads is written first in the same call, every output element is
written), and a workspace smaller than the plan asks for is refused before
anything runs.  Both cache formats, whole and split requests."""
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from decode_attention_absorbed_amd import binding as bnd  # noqa: E402
from workloads import make_inputs, make_inputs_fp8  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def setup(kv, dev, num_cus):
    if kv == "bf16":
        x = make_inputs(3, 128, 2, 64, [3000, 700, 65], seed=71)
        t = x.to_torch(dev)
        plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)

        def run(**kw):
            return mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                                  x.softmax_scale, **kw)
    else:
        x = make_inputs_fp8(3, 128, 2, 64, [3000, 700, 65], seed=72)
        t = x.to_torch(dev)
        plan = bnd.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)

        def run(**kw):
            return bnd.mla_decode_fp8(plan, t["q_nope"], t["q_pe"], t["cache_codes"], t["cache_exps"],
                                      t["block_table"], t["seq_lens"], x.softmax_scale, **kw)
    return x, plan, run


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("num_cus", [1, 256])
def test_results_do_not_depend_on_buffer_contents(dev, kv, num_cus):
    x, plan, run = setup(kv, dev, num_cus)
    shape_o, shape_l = (x.batch, x.q_len, x.heads, 512), (x.batch, x.q_len, x.heads)
    need = plan.workspace_bytes
    if num_cus == 256:
        assert need > 0  # the longer requests are split
    results = []
    for fill in (0xFF, 0x00, 0x7B):  # NaN bytes, zeros, large finite halves and floats
        ws = torch.full((max(need, 1),), fill, dtype=torch.uint8, device=dev)
        out = torch.full(shape_o, float("nan") if fill == 0xFF else float(fill), dtype=torch.float32, device=dev)
        lse = torch.full(shape_l, float("nan") if fill == 0xFF else -float(fill), dtype=torch.float32, device=dev)
        o, l = run(out=out, lse=lse, workspace=ws if need else None)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(l).all(), f"fill {fill:#x}"
        results.append((o.clone(), l.clone()))
    for o, l in results[1:]:
        assert torch.equal(o, results[0][0]) and torch.equal(l, results[0][1])
    plan.destroy()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_small_workspace_is_refused(dev, kv):
    x, plan, run = setup(kv, dev, 256)
    need = plan.workspace_bytes
    assert need > 0
    out = torch.full((x.batch, x.q_len, x.heads, 512), 7.0, dtype=torch.float32, device=dev)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device=dev)
    with pytest.raises(mla.MLAError):
        run(out=out, workspace=ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
    plan.destroy()
