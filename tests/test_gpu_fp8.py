"""FP8-cache decode (HIP, through the C ABI) against the fp64 FP8 oracle on an MI355X.

Tolerance, derived from the arithmetic (the oracle module states the model):
the scores use the same E4M3 query codes and exactly scaled keys on both sides,
so lse differs only by fp32 rounding (bar: max-abs <= 1e-3, as for bf16, or the
worst-case rounding of a 576-term fp32 sum where scores are large).  The
output differs mainly because the kernel rounds the softmax weights to E4M3
before the PV product; ``fp8_weight_error_rms`` gives the root-mean-square
size of that error per element (pinned against a direct simulation of the
rounding to within 0.75-1.33x).  Bars: the L2 norm of the error is at most
1.25x the model's, every element is within 6 model standard deviations
(+ 1e-4 for fp32 rounding), and the relative L2 error is at most 3%.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from decode_attention_absorbed_amd import binding as bnd  # noqa: E402
from oracle import (  # noqa: E402
    dequantize_cache,
    dequantize_query,
    fp8_weight_error_rms,
    mla_decode_fp8_ref,
    quantize_query,
)
from workloads import (  # noqa: E402
    make_config_fp8,
    make_inputs_fp8,
    poison_tails_fp8,
    poison_unreferenced_fp8,
)

pytestmark = pytest.mark.gpu

LSE_MAX_ABS = 1e-3
RMS_FACTOR, SIGMAS, ABS_FLOOR, REL_L2_CAP = 1.25, 6.0, 1e-4, 0.03


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_gpu(x, dev, num_cus=0, seq_lens_dev=None, block_table=None, plan=None):
    t = x.to_torch(dev)
    if plan is None:
        plan = bnd.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    bt = t["block_table"] if block_table is None else block_table
    sl = t["seq_lens"] if seq_lens_dev is None else seq_lens_dev
    out, lse = bnd.mla_decode_fp8(plan, t["q_nope"], t["q_pe"], t["cache_codes"], t["cache_exps"], bt, sl, x.softmax_scale)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def oracle(x, idx=None):
    idx = np.arange(x.batch) if idx is None else np.asarray(idx)
    args = (x.q_nope_f64()[idx], x.q_pe_f64()[idx], x.cache_codes, x.cache_exps, x.block_table[idx], x.seq_lens[idx], x.softmax_scale)
    o, l = mla_decode_fp8_ref(*args)
    rms = fp8_weight_error_rms(*args)
    return o, l, rms, score_abs_max(x, idx)


def score_abs_max(x, idx):
    """Per row, scale * max_t sum_i |q_i k_ti| over its visible keys: the size
    of the terms the fp32 score sums add up (their rounding scales with it)."""
    codes, f = quantize_query(x.q_nope_f64()[idx], x.q_pe_f64()[idx])
    q = np.abs(dequantize_query(codes, f))
    cache = np.abs(dequantize_cache(x.cache_codes, x.cache_exps))
    out = np.zeros(q.shape[:-1])
    for i, b in enumerate(idx):
        L = int(x.seq_lens[b])
        t = np.arange(L)
        K = cache[x.block_table[b, t // x.page], t % x.page]
        for j in range(x.q_len):
            n = L - x.q_len + 1 + j
            out[i, j] = x.softmax_scale * (q[i, j] @ K[:n].T).max(axis=-1)
    return out


def compare(out, lse, ref_o, ref_l, rms, s_abs, what=""):
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    err = out - ref_o
    e_l = float(np.max(np.abs(lse - ref_l)))
    ratio = float(np.linalg.norm(err) / max(np.linalg.norm(rms), 1e-300))
    worst = float(np.max(np.abs(err) / (SIGMAS * rms + ABS_FLOOR)))
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref_o), 1e-300))
    print(
        f"{what}: out max-abs {np.max(np.abs(err)):.3e} rel-L2 {rel:.3e} | L2 / model {ratio:.3f} "
        f"| worst element / bar {worst:.3f} | lse max-abs {e_l:.3e}",
        flush=True,
    )
    # lse: 1e-3, or the worst-case rounding of a 576-term fp32 score sum,
    # 576 * 2^-24 of the sum of the terms' magnitudes, where scores are large
    # (|d lse| <= max_t |d s_t|)
    bar_l = np.maximum(LSE_MAX_ABS, 576 * 2.0**-24 * s_abs)
    assert np.all(np.abs(lse - ref_l) <= bar_l), f"{what}: lse max-abs {e_l}"
    assert ratio <= RMS_FACTOR, f"{what}: error L2 is {ratio:.2f}x the model's"
    assert worst <= 1.0, f"{what}: an element is {worst:.2f}x past its bar"
    assert rel <= REL_L2_CAP, f"{what}: relative L2 error {rel:.3f}"


SMALL = [
    # (batch, heads, q_len, page, lens)
    (2, 16, 1, 16, [37, 100]),
    (3, 128, 1, 64, [1, 64, 200]),
    (3, 128, 2, 64, [2, 65, 300]),
    (4, 64, 1, 32, [31, 32, 33, 257]),
    (2, 100, 1, 16, [129, 17]),
    (2, 64, 3, 128, [3, 400]),
    (5, 128, 1, 256, [1000, 1, 513, 64, 300]),
    (1, 32, 8, 16, [111]),
    (3, 128, 4, 16, [1000, 257, 31]),
    (2, 128, 8, 32, [700, 9]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}" for c in SMALL])
def test_fp8_small_cases(dev, case):
    B, H, q, P, lens = case
    x = make_inputs_fp8(B, H, q, P, lens, seed=200 + sum(lens))
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=str(case))


@pytest.mark.parametrize("num_cus", [1, 7, 256])
def test_fp8_forced_split_counts(dev, num_cus):
    x = make_inputs_fp8(3, 128, 2, 64, [1500, 700, 90], seed=25)
    out, lse = run_gpu(x, dev, num_cus=num_cus)
    compare(out, lse, *oracle(x), what=f"num_cus={num_cus}")


@pytest.mark.parametrize("q_len,page", [(1, 16), (2, 64)])
def test_fp8_many_short_requests(dev, q_len, page):
    """60 requests of 1..300 keys (16 heads, to keep the oracle's query
    quantization short) planned for 8 CUs: every workgroup runs several
    requests one after another, every request against the oracle."""
    rng = np.random.default_rng(7 + q_len)
    lens = rng.integers(q_len, 301, size=60).tolist()
    x = make_inputs_fp8(len(lens), 16, q_len, page, lens, seed=310 + q_len)
    plan = bnd.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page, 8)
    wg = plan.workgroups()
    assert (wg[:, 1] - wg[:, 0]).min() >= 3
    out, lse = run_gpu(x, dev, plan=plan)
    compare(out, lse, *oracle(x), what=f"60 short requests, q_len {q_len}, page {page}")


@pytest.mark.parametrize("name", ["tiny", "dsv3", "mtp", "mixed", "long", "mtp4", "mtp8"])
def test_fp8_named_workload_parity(dev, name):
    x = make_config_fp8(name)
    print(f"{name}: B={x.batch} H={x.heads} q_len={x.q_len} pages={x.num_pages}", flush=True)
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=f"{name}, all {x.batch} requests")


@pytest.mark.parametrize("num_cus", [1, 3])
def test_fp8_pieces_spanning_more_than_64_pages(dev, num_cus):
    # page 16: a piece of more than 1024 keys reads page ids past the 64 the
    # kernel keeps in a register (scalar loads from the block table)
    x = make_inputs_fp8(2, 128, 1, 16, [3000, 2100], seed=38)
    plan = bnd.mla_decode_fp8_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    segs = plan.segments()
    assert max(-(-int(e) // 16) - int(s) // 16 for _, s, e, _ in segs) > 64
    out, lse = run_gpu(x, dev, plan=plan)
    compare(out, lse, *oracle(x), what=f"num_cus={num_cus}")


@pytest.mark.parametrize("page,lens", [(512, [5000, 700, 513]), (4096, [9000, 4097, 1])], ids=["P512", "P4096"])
def test_fp8_large_page_sizes(dev, page, lens):
    x = make_inputs_fp8(len(lens), 128, 1, page, lens, seed=39 + page)
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=f"page {page}")


@pytest.mark.parametrize("num_cus", [1, 256])
def test_fp8_out_of_range_page_ids_give_nan_in_exactly_their_requests(dev, num_cus):
    x = make_inputs_fp8(3, 128, 2, 16, [400, 200, 333], seed=36)
    good_o, good_l = run_gpu(x, dev, num_cus=num_cus)
    bt = x.block_table.copy()
    # (make_inputs shuffles the requests: index the pages request 0 really has)
    bt[0, (int(x.seq_lens[0]) - 1) // x.page // 2] = x.num_pages + 7  # past the pool
    bt[2, 0] = -3
    out, lse = run_gpu(x, dev, num_cus=num_cus, block_table=torch.from_numpy(bt).to(dev))
    for b in (0, 2):
        assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b]))
    np.testing.assert_array_equal(out[1], good_o[1])
    np.testing.assert_array_equal(lse[1], good_l[1])


def test_fp8_page_permutation_is_bitwise_invariant(dev):
    x = make_inputs_fp8(3, 128, 1, 16, [300, 47, 129], seed=29)
    o1, l1 = run_gpu(x, dev)
    perm = np.random.default_rng(1).permutation(x.num_pages)
    codes2 = np.empty_like(x.cache_codes)
    exps2 = np.empty_like(x.cache_exps)
    codes2[perm] = x.cache_codes
    exps2[perm] = x.cache_exps
    x.block_table = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    x.cache_codes, x.cache_exps = codes2, exps2
    o2, l2 = run_gpu(x, dev)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_fp8_nan_tails_and_unreferenced_pages_never_reach_the_output(dev):
    x = make_inputs_fp8(3, 128, 2, 64, [100, 65, 7], seed=31, extra_pages=3)
    o1, l1 = run_gpu(x, dev)
    poison_tails_fp8(x)
    poison_unreferenced_fp8(x)
    o2, l2 = run_gpu(x, dev)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_fp8_single_visible_key_returns_its_latent_row(dev):
    x = make_inputs_fp8(2, 128, 1, 16, [1, 1], seed=34)
    out, lse = run_gpu(x, dev)
    ref_o, ref_l, _, _ = oracle(x)
    cache = dequantize_cache(x.cache_codes, x.cache_exps)
    for b in range(2):
        row = cache[x.block_table[b, 0], 0, :512]
        # one key, weight 1: P' rounds to 2^6 exactly, so out is the
        # dequantized row up to fp32 rounding of the weight (1 - p ~ 1e-7)
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(row, (128, 512)), rtol=2e-6, atol=1e-6)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=LSE_MAX_ABS)  # fp32 dot of 576 terms


def test_fp8_repeat_runs_are_bitwise_identical(dev):
    x = make_inputs_fp8(4, 128, 1, 64, [2000, 5, 640, 999], seed=33)
    a = run_gpu(x, dev)
    b = run_gpu(x, dev)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_fp8_plan_and_kernel_kinds_do_not_mix(dev):
    x = make_inputs_fp8(1, 16, 1, 16, [40], seed=35)
    t = x.to_torch(dev)
    p16 = mla.mla_decode_plan(x.seq_lens, 1, 16, 16)
    with pytest.raises(bnd.MLAError):
        bnd.mla_decode_fp8(p16, t["q_nope"], t["q_pe"], t["cache_codes"], t["cache_exps"], t["block_table"], t["seq_lens"], 0.1)
    p8 = bnd.mla_decode_fp8_plan(x.seq_lens, 1, 16, 16)
    cache_bf16 = torch.zeros((x.num_pages, 16, 576), dtype=torch.bfloat16, device=dev)
    with pytest.raises(bnd.MLAError):
        mla.mla_decode(p8, t["q_nope"], t["q_pe"], cache_bf16, t["block_table"], t["seq_lens"], 0.1)


def _pages_of(x, b, t0, t1):
    """(page, slot) pairs of keys t0 .. t1-1 of request b."""
    t = np.arange(t0, t1)
    return x.block_table[b, t // x.page], t % x.page


@pytest.mark.parametrize("part", ["rope", "c_kv"])
def test_fp8_one_query_part_alone_decides_the_scores(dev, part):
    # As for the bf16 cache: the other part of every query row is zero (its
    # MXFP8 blocks quantize to zero codes), so the scores come from the rope
    # dimensions alone (the rope part scaled by 4, exact in bf16) or from
    # the c_kv dimensions alone.
    for heads, lens, seed in ((128, [300, 97, 33], 23), (16, [260, 5], 24)):
        x = make_inputs_fp8(len(lens), heads, 2, 64, lens, seed=seed)
        if part == "rope":
            x.q_nope[:] = 0
            pe = x.q_pe.astype(np.uint32)
            nz = (pe & 0x7F80) != 0  # normal numbers: add 2 to the exponent
            x.q_pe = np.where(nz, pe + (2 << 7), pe).astype(np.uint16)
        else:
            x.q_pe[:] = 0
        out, lse = run_gpu(x, dev)
        compare(out, lse, *oracle(x), what=f"{part} part alone, {heads} heads")


def test_fp8_row_reference_moves_and_output_rescales(dev):
    # Keys from 256 on get 8x larger scale bytes' worth (+3): their scores
    # dwarf the first tiles' by far more than 2^32 in log2 units, so every
    # row's reference moves mid-piece and the accumulated output is rescaled.
    x = make_inputs_fp8(2, 128, 1, 64, [600, 450], seed=41)
    for b, L in enumerate(x.seq_lens):
        pg, sl = _pages_of(x, b, 256, int(L))
        x.cache_exps[pg, sl] += 3
    out, lse = run_gpu(x, dev, num_cus=1)  # one piece per request: the moves happen inside it
    compare(out, lse, *oracle(x), what="reference moves")


def test_fp8_scale_reference_moves(dev):
    # The first tile's scale bytes sit 70 below the rest (more than the 2^64
    # the PV scale operand may carry between tiles): when the second tile
    # arrives, the kernel's scale reference moves and the output accumulated
    # so far is rescaled.  Scores stay moderate (the first tile's are ~0).
    x = make_inputs_fp8(2, 64, 1, 64, [400, 130], seed=43)
    for b in range(2):
        pg, sl = _pages_of(x, b, 0, 64)
        x.cache_exps[pg, sl] = (x.cache_exps[pg, sl].astype(np.int32) - 70).astype(np.uint8)
    out, lse = run_gpu(x, dev, num_cus=1)
    compare(out, lse, *oracle(x), what="scale reference moves")


def test_fp8_one_million_key_request(dev):
    """One request of 1,048,576 keys (0.6 GB of codes, page 4096) split over
    the whole device, every row against the oracle."""
    x = make_inputs_fp8(1, 128, 1, 4096, [1 << 20], seed=402)
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what="2^20 keys, page 4096")
