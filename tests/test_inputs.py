"""The seeded input generator: determinism, row slicing, bf16 exactness and
the workload recipes (exact ignored-row counts, Zipf head mass).  CPU only."""
import numpy as np

import lce_inputs as li


def test_row_slices_match_full_draw():
    full = li.normal_rows(3000, 1500, 0.5, 0, li.KEY_W, True)
    part = li.normal_rows(3000, 1500, 0.5, 0, li.KEY_W, True, 1234, 2901)
    np.testing.assert_array_equal(full[1234:2901], part)
    again = li.normal_rows(3000, 1500, 0.5, 0, li.KEY_W, True)
    np.testing.assert_array_equal(full, again)


def test_bf16_rounding_is_exact_and_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.1415926, 1e-3], np.float32)
    r = li.round_to_bf16(x)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even one (1.0)
    assert r[1] == 1.0
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert r[2] == np.float32(1.0078125)
    assert abs(r[3] - x[3]) <= abs(x[3]) * 2.0 ** -8


def test_f16_rounding_is_exact_and_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -11, 1.0 + 3.0 * 2.0 ** -11, -3.1415926, 1e-3], np.float32)
    r = li.round_to_f16(x)
    # every value survives a round trip through binary16 unchanged
    np.testing.assert_array_equal(r.astype(np.float16).astype(np.float32), r)
    # 1 + 2^-11 is halfway between 1 and 1 + 2^-10: ties go to the even one (1.0)
    assert r[1] == 1.0
    # 1 + 3 * 2^-11 is halfway between 1 + 2^-10 and 1 + 2^-9: even is 1 + 2^-9
    assert r[2] == np.float32(1.0 + 2.0 ** -9)
    assert abs(r[3] - x[3]) <= abs(x[3]) * 2.0 ** -11
    w = li.normal_rows(50, 40, 0.3, 7, li.KEY_W, "f16")
    np.testing.assert_array_equal(w.astype(np.float16).astype(np.float32), w)


def test_ignored_counts_are_exact():
    for cfg, n_ign in ((li.TINY_F32, 26), (li.MID_BF16, 205),
                       (li.LARGE_VOCAB_BF16, 410), (li.NONE_BF16, 0)):
        t = li.targets(cfg.N, cfg.V, cfg.targets, cfg.ignore_frac, cfg.seed)
        assert t.dtype == np.int64 and t.shape == (cfg.N,)
        assert int((t == -100).sum()) == n_ign
        ok = t[t != -100]
        assert ok.min() >= 0 and ok.max() < cfg.V


def test_zipf_head_mass():
    rng = np.random.default_rng(1)
    k = li.zipf_ranks(200000, 128256, 1.1, rng)
    w = np.arange(1, 128257, dtype=np.float64) ** -1.1
    p0 = w[0] / w.sum()
    assert abs((k == 0).mean() - p0) < 0.005
    assert abs((k < 10).mean() - w[:10].sum() / w.sum()) < 0.005


def test_small_config_shapes_and_scales():
    d = li.lce_inputs(li.TINY_F32)
    assert d["X"].shape == (256, 64) and d["W"].shape == (1000, 64)
    assert d["b"].shape == (1000,) and d["u"] is None
    assert abs(d["W"].std() - 1 / 8) < 0.01 and abs(d["b"].std() - 0.1) < 0.02
    part = li.lce_inputs(li.TINY_F32, rows=slice(64, 128))
    np.testing.assert_array_equal(part["X"], d["X"][64:128])
    np.testing.assert_array_equal(part["t"], d["t"][64:128])
