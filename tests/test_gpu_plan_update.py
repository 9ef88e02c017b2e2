"""mla_decode_plan_update on an MI355X: a plan re-planned in place for new
lengths (same batch shape) gives exactly what a fresh plan gives, updates
are ordered on the stream (decodes enqueued before an update keep the old
schedule), and a refused update leaves the plan as it was; the same for the
FP8 kernel's plans."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from oracle import mla_decode_ref  # noqa: E402
from workloads import make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def decode(x, t, plan):
    return mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"], x.softmax_scale)


@pytest.mark.parametrize("num_cus", [0, 7])
def test_updates_match_fresh_plans_in_stream_order(dev, num_cus):
    H, q, P = 128, 2, 64
    xa = make_inputs(4, H, q, P, [3000, 700, 65, 2000], seed=61)
    xb = make_inputs(4, H, q, P, [100, 4000, 1500, 33], seed=62)
    xc = make_inputs(4, H, q, P, [2, 2, 9000, 2], seed=63)
    ta, tb, tc = xa.to_torch(dev), xb.to_torch(dev), xc.to_torch(dev)
    refs = {}
    for name, x, t in (("a", xa, ta), ("b", xb, tb), ("c", xc, tc)):
        fresh = mla.mla_decode_plan(x.seq_lens, q, H, P, num_cus)
        o, l = decode(x, t, fresh)
        torch.cuda.synchronize()
        refs[name] = (o.clone(), l.clone(), fresh.query(mla.binding.MLA_Q_NUM_PARTIALS))
        fresh.destroy()

    # one plan, re-planned between decodes with no synchronization in between
    plan = mla.mla_decode_plan(xa.seq_lens, q, H, P, num_cus)
    outs = []
    for name, x, t in (("a", xa, ta), ("b", xb, tb), ("c", xc, tc), ("a", xa, ta), ("c", xc, tc)):
        if outs:
            plan.update(x.seq_lens)
        assert plan.query(mla.binding.MLA_Q_NUM_PARTIALS) == refs[name][2]
        outs.append((name,) + decode(x, t, plan))
    torch.cuda.synchronize()
    for name, o, l in outs:
        assert torch.equal(o, refs[name][0]) and torch.equal(l, refs[name][1]), name

    # and the updated plan's output against the oracle
    ro, rl = mla_decode_ref(xc.q_nope_f64(), xc.q_pe_f64(), xc.cache_f64(), xc.block_table, xc.seq_lens,
                            xc.softmax_scale)
    o = outs[-1][1].cpu().double().numpy()
    assert np.max(np.abs(o - ro)) <= 1e-2
    assert np.max(np.abs(outs[-1][2].cpu().double().numpy() - rl)) <= 1e-3
    plan.destroy()


def test_refused_update_leaves_the_plan_unchanged(dev):
    x = make_inputs(2, 64, 1, 16, [500, 90], seed=64)
    t = x.to_torch(dev)
    plan = mla.mla_decode_plan(x.seq_lens, 1, 64, 16, 256)
    o1, l1 = decode(x, t, plan)
    with pytest.raises(mla.MLAError):
        plan.update([0, 90])  # shorter than q_len
    with pytest.raises(mla.MLAError):
        plan.update([1 << 25, 90])  # beyond 2^24
    o2, l2 = decode(x, t, plan)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    plan.destroy()


def test_fp8_plan_update_matches_fresh_plans(dev):
    """The FP8 kernel's plans (64-key tiles) are re-planned the same way."""
    from workloads import make_inputs_fp8

    H, q, P = 128, 2, 64
    xs = [make_inputs_fp8(3, H, q, P, lens, seed=s) for lens, s in (([3000, 700, 65], 65), ([90, 5000, 1200], 66),
                                                                      ([2, 2, 8000], 67))]
    ts = [x.to_torch(dev) for x in xs]

    def run(x, t, plan):
        return mla.binding.mla_decode_fp8(plan, t["q_nope"], t["q_pe"], t["cache_codes"], t["cache_exps"],
                                          t["block_table"], t["seq_lens"], x.softmax_scale)

    refs = []
    for x, t in zip(xs, ts):
        fresh = mla.binding.mla_decode_fp8_plan(x.seq_lens, q, H, P, 0)
        o, l = run(x, t, fresh)
        torch.cuda.synchronize()
        refs.append((o.clone(), l.clone()))
        fresh.destroy()
    plan = mla.binding.mla_decode_fp8_plan(xs[0].seq_lens, q, H, P, 0)
    outs = []
    for i in (0, 1, 2, 0):
        if outs:
            plan.update(xs[i].seq_lens)
        outs.append((i,) + run(xs[i], ts[i], plan))
    torch.cuda.synchronize()
    for i, o, l in outs:
        assert torch.equal(o, refs[i][0]) and torch.equal(l, refs[i][1]), i
    plan.destroy()
