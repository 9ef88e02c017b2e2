"""HIP path against the fp64 oracle on an MI355X (through the C ABI).

Tolerances (the bar the build is held to): out max-abs <= 1e-2 and
relative L2 <= 5e-3 over the compared tensor; lse max-abs <= 1e-3.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import decode_attention_absorbed_amd as mla  # noqa: E402
from decode_attention_absorbed_amd import binding as bnd  # noqa: E402
from oracle import mla_decode_ref  # noqa: E402
from workloads import CONFIGS, make_config, make_inputs, poison_tails, poison_unreferenced  # noqa: E402

pytestmark = pytest.mark.gpu

OUT_MAX_ABS, OUT_REL_L2, LSE_MAX_ABS = 1e-2, 5e-3, 1e-3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def run_gpu(x, dev, num_cus=0, seq_lens_dev=None, block_table=None, plan=None):
    t = x.to_torch(dev)
    if plan is None:
        plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    bt = t["block_table"] if block_table is None else block_table
    sl = t["seq_lens"] if seq_lens_dev is None else seq_lens_dev
    out, lse = mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], bt, sl, x.softmax_scale)
    torch.cuda.synchronize()
    return out.cpu().double().numpy(), lse.cpu().double().numpy()


def oracle(x, idx=None):
    """fp64 reference for the requests in idx (all if None)."""
    idx = np.arange(x.batch) if idx is None else np.asarray(idx)
    cache = x.cache_f64()
    o, l = mla_decode_ref(x.q_nope_f64()[idx], x.q_pe_f64()[idx], cache, x.block_table[idx], x.seq_lens[idx], x.softmax_scale)
    return o, l


def compare(out, lse, ref_o, ref_l, what=""):
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)), f"{what}: non-finite output"
    e_o = float(np.max(np.abs(out - ref_o)))
    rel = float(np.linalg.norm(out - ref_o) / max(np.linalg.norm(ref_o), 1e-300))
    e_l = float(np.max(np.abs(lse - ref_l)))
    print(f"{what}: out max-abs {e_o:.3e} rel-L2 {rel:.3e} lse max-abs {e_l:.3e}", flush=True)
    assert e_o <= OUT_MAX_ABS, f"{what}: out max-abs {e_o}"
    assert rel <= OUT_REL_L2, f"{what}: out rel-L2 {rel}"
    assert e_l <= LSE_MAX_ABS, f"{what}: lse max-abs {e_l}"


# ---- small cases spanning several tiles and ragged tails ----------------------------------

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
    # full head count with long drafts: 4 and 8 row blocks of 128 rows per request
    (3, 128, 4, 16, [1000, 257, 31]),
    (2, 128, 8, 32, [700, 9]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}q{c[2]}P{c[3]}" for c in SMALL])
def test_small_cases(dev, case):
    B, H, q, P, lens = case
    x = make_inputs(B, H, q, P, lens, seed=100 + sum(lens))
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=str(case))


@pytest.mark.parametrize("num_cus", [1, 2, 7, 64, 256, 1024])
def test_forced_split_counts_agree(dev, num_cus):
    x = make_inputs(3, 128, 2, 64, [1500, 700, 90], seed=5)
    out, lse = run_gpu(x, dev, num_cus=num_cus)
    compare(out, lse, *oracle(x), what=f"num_cus={num_cus}")
    # Different splits round P to bf16 against different running maxima, so the
    # outputs agree to the bf16 level, not bitwise; the lse (fp32 sums) agrees closely.
    base_o, base_l = run_gpu(x, dev, num_cus=1)
    assert np.max(np.abs(out - base_o)) < OUT_MAX_ABS
    assert np.linalg.norm(out - base_o) / np.linalg.norm(base_o) < OUT_REL_L2
    assert np.max(np.abs(lse - base_l)) < 1e-5


@pytest.mark.parametrize("L,num_cus", [(1024, 8), (8192, 256)], ids=["few-pieces", "many-pieces"])
def test_both_combine_kernels(dev, L, num_cus):
    # at most 16 pieces per request take the one-wave-per-row combine, more the
    # four-waves-per-row one; both must merge to the oracle
    x = make_inputs(2, 128, 1, 64, [L, L // 2], seed=17)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    pieces = plan.query(bnd.MLA_Q_NUM_PARTIALS)
    assert (pieces <= 2 * 16) if L == 1024 else (pieces > 2 * 16)
    out, lse = run_gpu(x, dev, plan=plan)
    compare(out, lse, *oracle(x), what=f"L={L} num_cus={num_cus} pieces={pieces}")


# ---- the five named workloads at full size, every request against the oracle ------------


@pytest.mark.parametrize("name", ["tiny", "dsv3", "mtp", "mixed", "long"])
def test_named_workload_parity(dev, name):
    x = make_config(name)
    print(f"{name}: B={x.batch} H={x.heads} q_len={x.q_len} pages={x.num_pages}", flush=True)
    out, lse = run_gpu(x, dev)
    ref_o, ref_l = oracle(x)
    compare(out, lse, ref_o, ref_l, what=f"{name}, all {x.batch} requests")


# ---- invariants ---------------------------------------------------------------------------


def test_page_permutation_is_bitwise_invariant(dev):
    x = make_inputs(3, 128, 1, 16, [300, 47, 129], seed=9)
    o1, l1 = run_gpu(x, dev)
    rng = np.random.default_rng(1)
    perm = rng.permutation(x.num_pages)
    cache2 = np.empty_like(x.cache)
    cache2[perm] = x.cache
    bt2 = np.where(x.block_table >= 0, perm[np.maximum(x.block_table, 0)], -1).astype(np.int32)
    x.cache, x.block_table = cache2, bt2
    o2, l2 = run_gpu(x, dev)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_nan_tails_and_unreferenced_pages_never_reach_the_output(dev):
    x = make_inputs(3, 128, 2, 64, [100, 65, 7], seed=11, extra_pages=3)
    o1, l1 = run_gpu(x, dev)
    poison_tails(x)
    poison_unreferenced(x)
    o2, l2 = run_gpu(x, dev)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(l2))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    compare(o2, l2, *oracle(x), what="poisoned")


def test_mtp_queries_match_single_query_runs(dev):
    x = make_inputs(2, 128, 2, 64, [333, 64], seed=12)
    o, l = run_gpu(x, dev)
    x0 = make_inputs(2, 128, 1, 64, [332, 63], seed=12, draw_values=False)
    x0.q_nope, x0.q_pe, x0.cache, x0.num_pages = x.q_nope[:, :1].copy(), x.q_pe[:, :1].copy(), x.cache, x.num_pages
    x0.block_table = x.block_table[:, : x0.block_table.shape[1]].copy()
    o0, l0 = run_gpu(x0, dev)
    assert np.max(np.abs(o[:, 0] - o0[:, 0])) < 1e-4 and np.max(np.abs(l[:, 0] - l0[:, 0])) < 1e-4
    x1 = make_inputs(2, 128, 1, 64, [333, 64], seed=12, draw_values=False)
    x1.q_nope, x1.q_pe, x1.cache, x1.num_pages, x1.block_table = x.q_nope[:, 1:].copy(), x.q_pe[:, 1:].copy(), x.cache, x.num_pages, x.block_table
    o1, l1 = run_gpu(x1, dev)
    assert np.max(np.abs(o[:, 1] - o1[:, 0])) < 1e-4 and np.max(np.abs(l[:, 1] - l1[:, 0])) < 1e-4


@pytest.mark.parametrize("part", ["rope", "c_kv"])
def test_one_query_part_alone_decides_the_scores(dev, part):
    # The other part of every query row is zero, so the scores come from the
    # rope dimensions (512..575) alone, or from the c_kv dimensions alone;
    # the query's rope part is scaled by 4 (exact in bf16) so that its
    # scores spread as widely as the c_kv part's.  Rows of both row blocks
    # of every wave, 16- and 128-head requests, ragged tiles, two query tokens.
    for heads, lens, seed in ((128, [300, 97, 33], 21), (16, [260, 5], 22)):
        x = make_inputs(len(lens), heads, 2, 64, lens, seed=seed)
        if part == "rope":
            x.q_nope[:] = 0
            pe = x.q_pe.astype(np.uint32)
            nz = (pe & 0x7F80) != 0  # normal numbers: add 2 to the exponent
            x.q_pe = np.where(nz, pe + (2 << 7), pe).astype(np.uint16)
        else:
            x.q_pe[:] = 0
        out, lse = run_gpu(x, dev)
        compare(out, lse, *oracle(x), what=f"{part} part alone, {heads} heads")


def test_repeat_runs_are_bitwise_identical(dev):
    x = make_inputs(4, 128, 1, 64, [2000, 5, 640, 999], seed=13)
    t = x.to_torch(dev)
    plan = mla.mla_decode_plan(x.seq_lens, 1, 128, 64)
    a = mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"], x.softmax_scale)
    b = mla.mla_decode(plan, t["q_nope"], t["q_pe"], t["cache"], t["block_table"], t["seq_lens"], x.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_single_visible_key_returns_its_latent_row(dev):
    x = make_inputs(2, 128, 1, 16, [1, 1], seed=14)
    out, lse = run_gpu(x, dev)
    for b in range(2):
        row = x.cache_f64()[x.block_table[b, 0], 0]
        # out = the bf16 c_kv row exactly (one key, weight 1)
        np.testing.assert_allclose(out[b, 0], np.broadcast_to(row[:512], (128, 512)), rtol=0, atol=1e-6)
        s = x.softmax_scale * (np.concatenate([x.q_nope_f64()[b, 0], x.q_pe_f64()[b, 0]], axis=1) @ row)
        np.testing.assert_allclose(lse[b, 0], s, rtol=0, atol=1e-3)


@pytest.mark.parametrize("num_cus", [1, 256])  # request 1 whole, and split (NaN through the combine)
def test_device_length_mismatch_is_loud(dev, num_cus):
    x = make_inputs(2, 16, 1, 16, [40, 170], seed=15)
    wrong = torch.tensor([40, 169], dtype=torch.int32, device=dev)
    out, lse = run_gpu(x, dev, num_cus=num_cus, seq_lens_dev=wrong)
    assert np.all(np.isfinite(out[0])) and np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))


@pytest.mark.parametrize("num_cus", [1, 256])  # requests whole, and split (NaN through the combine)
def test_out_of_range_page_ids_give_nan_in_exactly_their_requests(dev, num_cus):
    # entries the plan needs hold ids outside [0, num_pages): the kernel never
    # follows them (page 0 is read instead, no fault) and the requests that
    # hold them end as NaN, out and lse; every other request is bit-identical
    x = make_inputs(3, 128, 2, 16, [400, 200, 333], seed=16)
    good_o, good_l = run_gpu(x, dev, num_cus=num_cus)
    bt = x.block_table.copy()
    # (make_inputs shuffles the requests: index the pages request 0 really has)
    bt[0, (int(x.seq_lens[0]) - 1) // x.page // 2] = x.num_pages + 7  # past the pool
    bt[2, 0] = -3  # negative
    out, lse = run_gpu(x, dev, num_cus=num_cus, block_table=torch.from_numpy(bt).to(dev))
    for b in (0, 2):
        assert np.all(np.isnan(out[b])) and np.all(np.isnan(lse[b]))
    np.testing.assert_array_equal(out[1], good_o[1])
    np.testing.assert_array_equal(lse[1], good_l[1])


@pytest.mark.parametrize("num_cus", [1, 3])
def test_pieces_spanning_more_than_64_pages(dev, num_cus):
    # page 16: a piece of more than 1024 keys reads page ids past the 64 the
    # kernel keeps in a register (scalar loads from the block table)
    x = make_inputs(2, 128, 1, 16, [3000, 2100], seed=18)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, num_cus)
    segs = plan.segments()
    assert max(-(-int(e) // 16) - int(s) // 16 for _, s, e, _ in segs) > 64
    out, lse = run_gpu(x, dev, plan=plan)
    compare(out, lse, *oracle(x), what=f"num_cus={num_cus}, pieces of up to {max(int(e) - int(s) for _, s, e, _ in segs)} keys")


@pytest.mark.parametrize("page,lens", [(512, [5000, 700, 513]), (1024, [3000, 1025]), (4096, [9000, 4097, 1])],
                         ids=["P512", "P1024", "P4096"])
def test_large_page_sizes(dev, page, lens):
    x = make_inputs(len(lens), 128, 1, page, lens, seed=19 + page)
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=f"page {page}")


# ---- more draft tokens (q_len 4 and 8 at full head count), every request -----------------


@pytest.mark.parametrize("name", ["mtp4", "mtp8"])
def test_long_draft_workloads(dev, name):
    x = make_config(name)
    out, lse = run_gpu(x, dev)
    ref_o, ref_l = oracle(x)
    compare(out, lse, ref_o, ref_l, what=f"{name}, all {x.batch} requests")


# ---- many short requests: several pieces per workgroup ------------------------------------


@pytest.mark.parametrize("q_len,page", [(1, 16), (2, 64)])
def test_many_short_requests(dev, q_len, page):
    """400 requests of 1..300 keys planned for 64 CUs: every workgroup runs
    several requests one after another (query reload, stage reuse and the
    barrier between pieces), every request against the oracle."""
    rng = np.random.default_rng(7 + q_len)
    lens = rng.integers(q_len, 301, size=400).tolist()
    x = make_inputs(len(lens), 128, q_len, page, lens, seed=300 + q_len)
    plan = mla.mla_decode_plan(x.seq_lens, x.q_len, x.heads, x.page, 64)
    wg = plan.workgroups()
    assert (wg[:, 1] - wg[:, 0]).min() >= 3  # several pieces per workgroup
    out, lse = run_gpu(x, dev, plan=plan)
    compare(out, lse, *oracle(x), what=f"400 short requests, q_len {q_len}, page {page}")


# ---- one request of 2^20 keys ---------------------------------------------------------------


@pytest.mark.parametrize("page", [16, 4096])
def test_one_million_key_request(dev, page):
    """One request of 1,048,576 keys (1.2 GB of cache) split over the whole
    device: pieces of 128 tiles, 256 partials merged by the combine, page ids
    up to 65535 (page 16: 256 pages per piece, nearly all looked up past the
    first 64), every row against the oracle."""
    x = make_inputs(1, 128, 1, page, [1 << 20], seed=401)
    print(f"page {page}: {x.num_pages} pages", flush=True)
    out, lse = run_gpu(x, dev)
    compare(out, lse, *oracle(x), what=f"2^20 keys, page {page}")
