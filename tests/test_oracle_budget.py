"""Pins for the per-layer update budgets (oracle.budget) and their host
entry point fb_layer_budgets (host logic: no GPU)."""

import ctypes as C
import math

import numpy as np
import pytest

from oracle import budget as B


def test_half_gaussians_meet_at_the_peak_layer():
    g = B.layer_shape(21, 10.0, 2.0, 4.0)
    assert g[10] == 1.0
    assert g[8] == math.exp(-0.5) and g[14] == math.exp(-0.5)     # one width each side
    assert g[6] == math.exp(-2.0) and g[18] == math.exp(-2.0)
    assert (np.diff(g[:11]) > 0).all() and (np.diff(g[10:]) < 0).all()


def test_equal_widths_are_symmetric_about_mu():
    g = B.layer_shape(32, 15.5, 5.0, 5.0)
    np.testing.assert_array_equal(g, g[::-1])


def test_ratios_hit_the_mean_and_the_floor():
    for mean, floor, mu, sl, sr in ((0.16, 0.04, 15.5, 6.0, 4.0), (0.25, 0.1, 5.0, 2.0, 8.0),
                                    (0.16, 0.16, 10.0, 3.0, 3.0)):
        r = B.layer_ratios(32, mean, floor, mu, sl, sr)
        assert abs(r.mean() - mean) < 1e-15
        assert r.min() >= floor - 1e-15
        if floor < mean:                          # a peak exists: at the layer nearest mu
            assert abs(np.argmax(r) - mu) <= 0.5
    # floor == mean: every layer at the mean
    np.testing.assert_allclose(B.layer_ratios(8, 0.2, 0.2, 3.0, 1.0, 1.0), 0.2, rtol=1e-15)


def test_counts_round_half_up_and_clamp():
    assert B.layer_counts(10, [0.04, 0.05, 0.06, 0.149, 0.15]).tolist() == [0, 1, 1, 1, 2]
    assert B.layer_counts(10, [-0.3, 1.7]).tolist() == [0, 10]
    r = B.layer_ratios(32, 0.16, 0.04, 15.5, 6.0, 4.0)
    n = B.layer_counts(1024, r)
    assert abs(n.mean() / 1024 - 0.16) < 1e-3


@pytest.mark.parametrize("params", [
    (32, 1024, 0.16, 0.04, 15.5, 6.0, 4.0),
    (32, 1024, 0.25, 0.25, 15.5, 6.0, 4.0),
    (24, 4096, 0.2, 0.01, 3.0, 1.5, 9.0),
    (1, 100, 0.3, 0.1, 0.0, 1.0, 1.0),
    (80, 777, 0.12, 0.02, 50.0, 20.0, 7.5),
])
def test_host_entry_point_matches_bit_for_bit(params):
    import block_diffusion_attention_amd as fb
    lib = fb.load()
    n_layers, n_tok, mean, floor, mu, sl, sr = params
    ratios = (C.c_double * n_layers)()
    counts = (C.c_int32 * n_layers)()
    st = lib.fb_layer_budgets(n_layers, n_tok, mean, floor, mu, sl, sr, ratios, counts)
    assert st == 0
    r = B.layer_ratios(n_layers, mean, floor, mu, sl, sr)
    assert list(ratios) == r.tolist()
    assert list(counts) == B.layer_counts(n_tok, r).tolist()


def test_host_entry_point_rejects():
    import block_diffusion_attention_amd as fb
    lib = fb.load()
    counts = (C.c_int32 * 4)()
    good = (4, 100, 0.16, 0.04, 1.5, 1.0, 1.0)
    assert lib.fb_layer_budgets(*good, None, counts) == 0
    for i, bad in ((0, 0), (1, -1), (2, 0.03), (2, 1.5), (3, -0.1), (5, 0.0), (6, -1.0),
                   (4, float("nan"))):
        p = list(good)
        p[i] = bad
        assert lib.fb_layer_budgets(*p, None, counts) == 1, (i, bad)
    assert lib.fb_layer_budgets(*good, None, None) == 1


def test_taus_hand_values():
    # base 4 at the mean ratio 0.16, B = 16 (never = 17):
    # 0.64 / r: 0.16 -> 4, 0.32 -> 2, 0.08 -> 8, 0.04 -> 16, 0 -> 17 (no
    # budget), 0.64 -> 1, 0.01 -> 64 clamped to 17, 0.11 -> 5.82 rounds to 6
    r = [0.16, 0.32, 0.08, 0.04, 0.0, 0.64, 0.01, 0.11]
    assert B.layer_taus(r, 16, 4, 0.16).tolist() == [4, 2, 8, 16, 17, 1, 17, 6]
    assert B.layer_taus([1.0, 0.5], 4, 3, 0.9).tolist() == [3, 5]       # 2.7 -> 3, 5.4 -> 5


def test_taus_fall_as_the_budget_grows():
    r = B.layer_ratios(32, 0.16, 0.04, 15.5, 6.4, 4.0)
    t = B.layer_taus(r, 16, 4, 0.16)
    order = np.argsort(r)
    assert (np.diff(t[order]) <= 0).all()            # larger budget -> no larger tau
    assert t[np.argmax(r)] < 4 < t[np.argmin(r)]
    # a uniform schedule keeps the base threshold in every layer
    assert (B.layer_taus(np.full(8, 0.16), 16, 4, 0.16) == 4).all()


def test_taus_host_entry_point_matches_bit_for_bit():
    import block_diffusion_attention_amd as fb
    r = B.layer_ratios(32, 0.16, 0.04, 15.5, 6.4, 4.0)
    for block, base in ((16, 4), (8, 2), (4, 2), (16, 1)):
        assert fb.fb_layer_taus(block, base, 0.16, r) == B.layer_taus(r, block, base, 0.16).tolist()
    odd = [0.16, 0.32, 0.08, 0.04, 0.0, 0.64, 0.01, 0.11, -0.5, 1e-300]
    assert fb.fb_layer_taus(16, 4, 0.16, odd) == B.layer_taus(odd, 16, 4, 0.16).tolist()


def test_taus_host_entry_point_rejects():
    import block_diffusion_attention_amd as fb
    lib = fb.load()
    r = (C.c_double * 3)(0.1, 0.2, 0.3)
    t = (C.c_int32 * 3)()
    assert lib.fb_layer_taus(3, 16, 4, 0.16, r, t) == 0
    for args in ((0, 16, 4, 0.16, r, t), (3, 0, 4, 0.16, r, t), (3, 16, 0, 0.16, r, t),
                 (3, 16, 4, 0.0, r, t), (3, 16, 4, 1.5, r, t), (3, 16, 4, float("nan"), r, t),
                 (3, 16, 4, 0.16, None, t), (3, 16, 4, 0.16, r, None)):
        assert lib.fb_layer_taus(*args) == 1, args
    bad = (C.c_double * 3)(0.1, float("inf"), 0.3)
    assert lib.fb_layer_taus(3, 16, 4, 0.16, bad, t) == 1
