"""The two O-rescale forms of the bf16 decode (mla_decode_variant) against the
fp64 oracle, on an MI355X through the C ABI.

MLA_RESCALE_POW2 is the power-of-two (AMLA) form of the online softmax's
reference: the Huawei report on DeepSeek V3/R1 deployment on Ascend servers,
section 6.1 (the AMLA bullet), turns O's multiplicative rescale into an
exponent add.  Both forms compute the same softmax, so both are held to the
bar of test_gpu_parity.py against the oracle; MLA_RESCALE_LAZY through this
entry point is the kernel mla_decode runs, so it must match it bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from oracle import mla_decode_ref  # noqa: E402
from workloads import bf16_bits_to_f64, make_config, make_inputs, to_bf16_bits  # noqa: E402

pytestmark = pytest.mark.gpu

OUT_MAX_ABS, OUT_REL_L2, LSE_MAX_ABS = 1e-2, 5e-3, 1e-3
VARIANTS = {"lazy": mla.MLA_RESCALE_LAZY, "pow2": mla.MLA_RESCALE_POW2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_variant(x, dev, variant, num_cus=0):
    t = x.to_torch(dev)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    events = torch.zeros(1, dtype=torch.int32, device=dev)
    out, lse = mla.mla_decode_variant(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                                      x.softmax_scale, variant=variant, rescale_events=events)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy(), int(events.item())


def compare_oracle(x, out, lse, what):
    ref_o, ref_l = mla_decode_ref(x.q_nope_f64(), x.q_pe_f64(), x.cache_f64(), x.block_table, x.seq_lens,
                                  x.softmax_scale)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    e_o = float(np.max(np.abs(out - ref_o)))
    rel = float(np.linalg.norm(out - ref_o) / np.linalg.norm(ref_o))
    e_l = float(np.max(np.abs(lse - ref_l)))
    print(f"{what}: out max-abs {e_o:.3e} rel-L2 {rel:.3e} lse max-abs {e_l:.3e}", flush=True)
    assert e_o <= OUT_MAX_ABS and rel <= OUT_REL_L2 and e_l <= LSE_MAX_ABS, what


def rising_scores(x, steps=((1 / 3, 8.0), (2 / 3, 64.0))):
    """Scales the rope part (dims 512..575) of each request's later keys by
    powers of two, in place: from fraction f of the sequence on, by g.  The
    row maxima of the scores then jump by far more than 2^8 (in base-2 units)
    partway through every request, so the lazy reference must move after O
    has accumulated.  The values (dims 0..511) are untouched."""
    pe = bf16_bits_to_f64(x.cache[:, :, 512:])
    for b in range(x.batch):
        L = int(x.seq_lens[b])
        tok = np.arange(L)
        pages = x.block_table[b, tok // x.page]
        slots = tok % x.page
        gain = np.ones(L)
        for frac, g in steps:
            gain[tok >= int(frac * L)] = g
        pe[pages, slots] *= gain[:, None]
    x.cache[:, :, 512:] = to_bf16_bits(pe)


CASES = [
    # (batch, heads, q_len, page, lens, seed)
    (3, 128, 1, 64, [1, 700, 2000], 51),
    (3, 128, 2, 16, [5, 300, 1500], 52),
    (2, 64, 4, 128, [900, 77], 53),
]


@pytest.mark.parametrize("name", list(VARIANTS))
@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}" for c in CASES])
@pytest.mark.parametrize("num_cus", [1, 256])
def test_variant_matches_oracle(dev, name, case, num_cus):
    B, H, q, P, lens, seed = case
    x = make_inputs(B, H, q, P, lens, seed=seed)
    out, lse, _ = run_variant(x, dev, VARIANTS[name], num_cus)
    compare_oracle(x, out, lse, f"{name} {case} num_cus={num_cus}")


@pytest.mark.parametrize("name", list(VARIANTS))
@pytest.mark.parametrize("num_cus", [1, 256])
def test_rescales_fire_and_stay_exact(dev, name, num_cus):
    x = make_inputs(3, 128, 2, 64, [3000, 1200, 700], seed=54)
    rising_scores(x)
    out, lse, events = run_variant(x, dev, VARIANTS[name], num_cus)
    print(f"{name} num_cus={num_cus}: {events} rescale events", flush=True)
    # every wave of every piece that spans a jump rescales at least once
    assert events >= 2 * 4 * 2, events
    compare_oracle(x, out, lse, f"{name} rising num_cus={num_cus}")


def test_lazy_variant_is_mla_decode(dev):
    x = make_inputs(4, 128, 2, 64, [3000, 700, 65, 2000], seed=55)
    rising_scores(x)
    t = x.to_torch(dev)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, 256)
    o1, l1 = mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"], x.softmax_scale)
    o2, l2 = mla.mla_decode_variant(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                                    x.softmax_scale, variant=mla.MLA_RESCALE_LAZY)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["dsv3", "mtp"])
def test_pow2_named_workloads(dev, name):
    x = make_config(name)
    out, lse, events = run_variant(x, dev, mla.MLA_RESCALE_POW2)
    print(f"{name}: {events} rescale events", flush=True)
    compare_oracle(x, out, lse, f"pow2 {name}")


def test_unknown_variant_is_refused(dev):
    x = make_inputs(1, 16, 1, 16, [40], seed=56)
    t = x.to_torch(dev)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page)
    with pytest.raises(mla.MLAError, match="variant"):
        mla.mla_decode_variant(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"],
                               x.softmax_scale, variant=2)


@pytest.mark.parametrize("num_cus", [7, 64, 256])
def test_pow2_splits_agree_to_the_partials_rounding(dev, num_cus):
    """With a power-of-two reference, a piece's weights are exact power-of-two
    multiples of the unsplit run's, so their bf16 rounding is the same: split
    and unsplit runs differ only by the fp16 storage of the partials (at most
    2^-11 of the largest |V| of the request, per element) and fp32 summation
    order.  The lazy form rounds P against each piece's own maximum, so it
    agrees only to the bf16 level (printed for comparison)."""
    x = make_inputs(3, 128, 2, 64, [3000, 1500, 700], seed=57)
    vmax = float(np.max(np.abs(x.cache_f64()[:, :, :512])))
    bound = 2.0**-11 * vmax + 1e-6
    diffs = {}
    for name in ("pow2", "lazy"):
        o1, l1, _ = run_variant(x, dev, VARIANTS[name], num_cus=1)
        o2, l2, _ = run_variant(x, dev, VARIANTS[name], num_cus=num_cus)
        diffs[name] = (float(np.max(np.abs(o2 - o1))), float(np.max(np.abs(l2 - l1))))
    print(f"num_cus={num_cus}: split vs whole max|d out| pow2 {diffs['pow2'][0]:.2e}, lazy {diffs['lazy'][0]:.2e}"
          f" (bound {bound:.2e}); max|d lse| pow2 {diffs['pow2'][1]:.2e}", flush=True)
    assert diffs["pow2"][0] <= bound
    assert diffs["pow2"][1] <= 1e-5
