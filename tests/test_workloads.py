"""The seeded input generator: shapes and structure of the five workloads."""
import numpy as np

from workloads import CONFIGS, config_lens, make_inputs, pages_needed, to_bf16_bits, bf16_bits_to_f64


def test_bf16_rounding_is_round_to_nearest_even():
    # 1 + 2^-8 lies exactly between two bf16 values: ties go to the even mantissa (1.0)
    x = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -2.5, 0.0, np.inf, np.nan], dtype=np.float32)
    bits = to_bf16_bits(x)
    back = bf16_bits_to_f64(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0 + 2.0**-6
    assert back[2] == -2.5 and back[3] == 0.0 and np.isinf(back[4]) and np.isnan(back[5])


def test_named_workload_structure():
    lens = config_lens("mixed")
    assert sorted(set(lens.tolist())) == [400, 20480]
    assert (lens == 20480).sum() == 26 and (lens == 400).sum() == 38
    assert sum(pages_needed(lens, 64)) == 8586
    mtp = config_lens("mtp")
    assert mtp.min() >= 1024 and mtp.max() <= 8192 and len(mtp) == 64
    assert config_lens("long").tolist() == [131072]
    assert config_lens("dsv3").tolist() == [4096] * 32
    assert sorted(config_lens("tiny").tolist()) == [37, 100]
    for name, B, q in (("mtp4", 32, 4), ("mtp8", 16, 8)):
        L = config_lens(name)
        assert len(L) == B and L.min() >= 1024 and L.max() <= 8192
        assert B * q * CONFIGS[name]["heads"] == 64 * 2 * 128  # the same query rows as "mtp"


def test_block_table_is_a_permutation_dealt_in_order():
    x = make_inputs(5, 4, 1, 16, [17, 1, 64, 65, 100], seed=3, draw_values=False)
    npg = pages_needed(x.seq_lens, 16)
    seen = np.concatenate([x.block_table[b, :n] for b, n in enumerate(npg)])
    assert sorted(seen.tolist()) == list(range(x.num_pages))
    for b, n in enumerate(npg):
        assert np.all(x.block_table[b, n:] == -1)


def test_seeded_determinism():
    a = make_inputs(2, 4, 2, 16, [20, 33], seed=9)
    b = make_inputs(2, 4, 2, 16, [20, 33], seed=9)
    for f in ("q_nope", "q_pe", "cache", "block_table", "seq_lens"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert set(CONFIGS) == {"tiny", "dsv3", "mtp", "mixed", "long", "mtp4", "mtp8"}


def test_prolog_inputs_structure_and_determinism():
    import numpy as np

    from workloads import bf16_bits_to_f64, make_prolog_inputs

    a = make_prolog_inputs(3, 2, 4, [5, 9, 17], seed=3, hidden=64)
    b = make_prolog_inputs(3, 2, 4, [5, 9, 17], seed=3, hidden=64)
    c = make_prolog_inputs(3, 2, 4, [5, 9, 17], seed=3)
    assert a.q_nope128.shape == (3, 2, 4, 128) and a.q_pe_raw.shape == (3, 2, 4, 64)
    assert a.w_uk_t.shape == (4, 512, 128) and a.w_uv.shape == (4, 128, 512) and a.w_o.shape == (64, 512)
    assert a.c_kv_raw.shape == (3, 2, 512) and a.k_pe_raw.shape == (3, 2, 64) and a.kv_norm_w.shape == (512,)
    assert a.rope_cos_sin.shape == (18, 64) and a.rope_cos_sin.dtype == np.float32
    for k in ("q_nope128", "q_pe_raw", "w_uk_t", "c_kv_raw", "kv_norm_w", "k_pe_raw", "w_uv", "w_o"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    # W_O is drawn last: asking for it leaves every other draw unchanged
    assert c.w_o is None and np.array_equal(c.w_uv, a.w_uv)
    # the RoPE table is cos then sin of p * 10000^(-2i/64)
    p, i = 7, 5
    ang = p * 10000.0 ** (-2 * i / 64)
    assert abs(a.rope_cos_sin[p, i] - np.cos(ang)) < 1e-6 and abs(a.rope_cos_sin[p, 32 + i] - np.sin(ang)) < 1e-6
    # W_UK^T's transpose is the [H, 128, 512] W_UK
    assert np.array_equal(a.w_uk_f64()[1, 3, 7], bf16_bits_to_f64(a.w_uk_t)[1, 7, 3])
