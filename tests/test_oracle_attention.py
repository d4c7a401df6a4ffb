"""Pins for oracle.attention: closed forms, the merge identity, libraries,
brute force and the grouped-query mapping.

Each check is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a transposed operand, a wrong head mapping, a log base) fails
one of them.
"""

import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle.attention import attn, attn_gqa, dense_step, kv_head_of, merge

rng = np.random.default_rng(1234)


def rand(*shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- closed forms

def test_two_key_hand_example():
    # q=[1,0], keys e1,e2, values e1,e2, scale 1: scores [1, 0];
    # Z = e + 1, A = [e, 1]/(e+1), L = ln(e+1).
    a, l = attn(np.array([[1.0, 0.0]]), np.eye(2), np.eye(2), 1.0)
    e = math.e
    assert a[0] == pytest.approx([e / (e + 1), 1 / (e + 1)], rel=1e-15)
    assert l[0] == pytest.approx(math.log(e + 1), rel=1e-15)


def test_zero_keys_give_mean_and_log_n():
    n, d = 37, 8
    v = rand(n, d)
    a, l = attn(rand(3, d), np.zeros((n, d)), v, 0.3)
    np.testing.assert_allclose(a, np.broadcast_to(v.mean(0), a.shape), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l, math.log(n), rtol=1e-15)


def test_constant_values_pass_through():
    c = rand(1, 6)
    a, _ = attn(rand(4, 6), rand(50, 6), np.repeat(c, 50, axis=0), 0.7)
    np.testing.assert_allclose(a, np.repeat(c, 4, axis=0), rtol=1e-13)


def test_single_key():
    q, k, v = rand(5, 8), rand(1, 8), rand(1, 8)
    a, l = attn(q, k, v, 0.25)
    np.testing.assert_allclose(a, np.repeat(v, 5, axis=0), rtol=1e-15)
    np.testing.assert_allclose(l, 0.25 * (q @ k[0]), rtol=1e-14)


def test_duplicated_keys_add_ln2():
    q, k, v = rand(3, 8), rand(20, 8), rand(20, 8)
    a1, l1 = attn(q, k, v, 0.5)
    a2, l2 = attn(q, np.concatenate([k, k]), np.concatenate([v, v]), 0.5)
    np.testing.assert_allclose(a2, a1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, l1 + math.log(2), rtol=1e-14)


def test_scale_enters_the_scores_not_the_output():
    # shifting all scores by a constant leaves A unchanged and moves L by it:
    # with k' = k + c*q/|q|^2 * t, every score of row q moves by scale*c*t.
    q = rand(1, 8)
    k, v = rand(30, 8), rand(30, 8)
    shift = 3.0
    k2 = k + shift * q / (q @ q.T)
    a1, l1 = attn(q, k, v, 0.5)
    a2, l2 = attn(q, k2, v, 0.5)
    np.testing.assert_allclose(a2, a1, rtol=1e-12)
    np.testing.assert_allclose(l2, l1 + 0.5 * shift, rtol=1e-13)


def test_empty_key_set():
    a, l = attn(rand(3, 4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(a == 0) and np.all(l == -np.inf)


# --------------------------------------------------------- libraries / brute

def test_matches_torch_sdpa_and_scipy_logsumexp():
    q, k, v = rand(6, 16), rand(90, 16), rand(90, 16)
    scale = 1 / math.sqrt(16)
    a, l = attn(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], scale=scale)[0].numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, scipy.special.logsumexp(scale * q @ k.T, axis=1), rtol=1e-14)


def test_brute_force_python_loops():
    q, k, v = rand(2, 3), rand(5, 3), rand(5, 2)
    scale = 0.9
    a, l = attn(q, k, v, scale)
    for i in range(2):
        s = [scale * sum(q[i][t] * k[j][t] for t in range(3)) for j in range(5)]
        z = sum(math.exp(x) for x in s)
        for c in range(2):
            want = sum(math.exp(s[j]) * v[j][c] for j in range(5)) / z
            assert a[i, c] == pytest.approx(want, rel=1e-13)
        assert l[i] == pytest.approx(math.log(z), rel=1e-14)


def test_large_scores_are_stable():
    q = np.full((1, 4), 100.0)
    k = rand(10, 4) * 10
    a, l = attn(q, k, rand(10, 4), 1.0)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(l))
    s = (q @ k.T)[0]
    assert l[0] == pytest.approx(scipy.special.logsumexp(s), rel=1e-14)


# ------------------------------------------------------------------- merge

def test_merge_reconstructs_full_attention():
    # FlashBlock core mechanism: the merge of the block-external and
    # block-internal pairs equals attention over the union of the key sets.
    q, k, v = rand(7, 32), rand(300, 32), rand(300, 32)
    a, l = attn(q, k, v, 0.2)
    for cut in (1, 17, 150, 299):
        ao, lo = attn(q, k[:cut], v[:cut], 0.2)
        ai, li = attn(q, k[cut:], v[cut:], 0.2)
        am, lm = merge(ao, lo, ai, li)
        np.testing.assert_allclose(am, a, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lm, l, rtol=1e-13)


def test_merge_any_partition_any_order():
    q, k, v = rand(4, 16), rand(400, 16), rand(400, 16)
    a, l = attn(q, k, v, 0.3)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(0, 401), size=7, replace=True))
        bounds = [0, *cuts.tolist(), 400]
        parts = [attn(q, k[lo:hi], v[lo:hi], 0.3) for lo, hi in zip(bounds[:-1], bounds[1:])]
        order = rng.permutation(len(parts))
        am, lm = parts[order[0]]
        for j in order[1:]:
            am, lm = merge(am, lm, *parts[j])
        np.testing.assert_allclose(am, a, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lm, l, rtol=1e-13)


def test_merge_is_symmetric_and_weights_by_exp_l():
    a1, a2 = rand(3, 5), rand(3, 5)
    l1, l2 = rand(3), rand(3)
    m12 = merge(a1, l1, a2, l2)
    m21 = merge(a2, l2, a1, l1)
    np.testing.assert_allclose(m12[0], m21[0], rtol=1e-15)
    w1, w2 = np.exp(l1), np.exp(l2)
    np.testing.assert_allclose(m12[0], (w1[:, None] * a1 + w2[:, None] * a2) / (w1 + w2)[:, None], rtol=1e-14)
    np.testing.assert_allclose(m12[1], np.log(w1 + w2), rtol=1e-14)


def test_merge_with_empty_sides():
    a1, l1 = rand(2, 3), rand(2)
    empty_a, empty_l = np.zeros((2, 3)), np.full(2, -np.inf)
    am, lm = merge(a1, l1, empty_a, empty_l)
    np.testing.assert_array_equal(am, a1)
    np.testing.assert_array_equal(lm, l1)
    am, lm = merge(empty_a, empty_l, empty_a, empty_l)
    assert np.all(am == 0) and np.all(lm == -np.inf)


def test_merge_far_apart_normalisers():
    a1, a2 = rand(1, 4), rand(1, 4)
    am, lm = merge(a1, np.array([800.0]), a2, np.array([0.0]))
    np.testing.assert_allclose(am, a1, rtol=1e-15)
    assert lm[0] == 800.0


# --------------------------------------------------------------------- GQA

def test_gqa_head_mapping_is_contiguous_groups():
    assert [kv_head_of(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head_of(h, 12, 12) for h in range(12)] == list(range(12))
    # each KV head carries its own constant value vector -> A reveals g(h)
    n_q, hq, hkv, d, n = 3, 8, 2, 4, 10
    v = np.zeros((n, hkv, d))
    for g in range(hkv):
        v[:, g, :] = g + 1
    a, _ = attn_gqa(rand(n_q, hq, d), rand(n, hkv, d), v, 0.5)
    for h in range(hq):
        np.testing.assert_allclose(a[:, h, :], h // (hq // hkv) + 1, rtol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    n_q, hq, hkv, d, n = 4, 8, 2, 16, 64
    q, k, v = rand(n_q, hq, d), rand(n, hkv, d), rand(n, hkv, d)
    a, l = attn_gqa(q, k, v, 0.25)
    krep = np.repeat(k, hq // hkv, axis=1)
    vrep = np.repeat(v, hq // hkv, axis=1)
    a2, l2 = attn_gqa(q, krep, vrep, 0.25)
    np.testing.assert_allclose(a, a2, rtol=1e-15)
    np.testing.assert_allclose(l, l2, rtol=1e-15)
    # and each head equals plain attention over its KV head
    for h in range(hq):
        ah, lh = attn(q[:, h], k[:, h // 4], v[:, h // 4], 0.25)
        np.testing.assert_allclose(a[:, h], ah, rtol=1e-15)


def test_dense_step_is_prefix_then_block():
    n_q, hq, hkv, d = 3, 4, 2, 8
    q = rand(n_q, hq, d)
    kp, vp = rand(40, hkv, d), rand(40, hkv, d)
    kb, vb = rand(n_q, hkv, d), rand(n_q, hkv, d)
    a, l = dense_step(q, kp, vp, kb, vb, 0.3)
    ao, lo = attn_gqa(q, kp, vp, 0.3)
    ai, li = attn_gqa(q, kb, vb, 0.3)
    am, lm = merge(ao, lo, ai, li)
    np.testing.assert_allclose(a, am, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l, lm, rtol=1e-13)
    # bidirectional block: query 0 sees the last block key
    kb2 = kb.copy()
    kb2[-1] += 5.0
    a2, _ = dense_step(q, kp, vp, kb2, vb, 0.3)
    assert not np.allclose(a2[0], a[0])
