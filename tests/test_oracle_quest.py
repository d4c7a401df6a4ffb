"""Pins for oracle.quest: page metadata, the page bound, top-k, the
selected/residual split and the union size."""

import json
import os

import numpy as np

from oracle import quest as Q
from oracle.attention import attn_gqa, merge

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(7)


def test_quest_hand_fixture():
    with open(os.path.join(GOLD, "quest_toy.json")) as f:
        g = json.load(f)
    k = np.array(g["keys"], dtype=np.float64)[:, None, :]          # [N, 1, d]
    kmin, kmax = Q.page_meta(k, g["page"])
    np.testing.assert_array_equal(kmin[0], g["kmin"])
    np.testing.assert_array_equal(kmax[0], g["kmax"])
    q = np.array(g["q"])[None, None, :]                              # [1, 1, d]
    u = Q.page_bound(q, kmin, kmax)
    np.testing.assert_array_equal(u[0, 0], g["bound"])
    assert Q.topk_pages(u, 2)[0, 0].tolist() == g["top2"]
    assert Q.topk_pages(u, 3)[0, 0].tolist() == g["top3"]


def test_page_meta_brute_force_with_ragged_last_page():
    k = rng.standard_normal((37, 2, 3))
    kmin, kmax = Q.page_meta(k, 8)
    assert kmin.shape == (2, 5, 3)
    for g in range(2):
        for p in range(5):
            toks = range(p * 8, min(37, p * 8 + 8))
            for j in range(3):
                assert kmin[g, p, j] == min(k[t, g, j] for t in toks)
                assert kmax[g, p, j] == max(k[t, g, j] for t in toks)


def test_bound_dominates_every_key_score_and_is_tight_for_one_token_pages():
    k = rng.standard_normal((64, 2, 8))
    q = rng.standard_normal((3, 4, 8))
    kmin, kmax = Q.page_meta(k, 8)
    u = Q.page_bound(q, kmin, kmax)
    for t in range(3):
        for h in range(4):
            g = h // 2
            for p in range(8):
                best = max(float(q[t, h] @ k[j, g]) for j in range(p * 8, p * 8 + 8))
                assert u[t, g, p] >= best - 1e-12
    # page of one token: bound = max over the group's heads of q.k
    kmin1, kmax1 = Q.page_meta(k, 1)
    u1 = Q.page_bound(q, kmin1, kmax1)
    for t in range(3):
        for g in range(2):
            want = np.max(q[t, 2 * g:2 * g + 2] @ k[:, g].T, axis=0)
            np.testing.assert_allclose(u1[t, g], want, rtol=1e-13, atol=1e-13)


def test_bound_sum_is_sequential_over_d():
    # an order-sensitive case: sequential float64 sum differs from pairwise
    d = 4
    kmin = np.array([[[1e16, 1.0, -1e16, 1.0]]])
    kmax = kmin.copy()
    q = np.ones((1, 1, d))
    u = Q.page_bound(q, kmin, kmax)
    seq = 0.0
    for x in (1e16, 1.0, -1e16, 1.0):
        seq = seq + x
    assert u[0, 0, 0] == seq == 1.0


def test_topk_matches_full_sort_and_breaks_ties_by_page():
    u = rng.integers(0, 5, size=(3, 2, 40)).astype(np.float64)   # many ties
    for k in (0, 1, 7, 40):
        sel = Q.topk_pages(u, k)
        for t in range(3):
            for g in range(2):
                want = sorted(sorted(range(40), key=lambda p: (-u[t, g, p], p))[:k])
                assert sel[t, g].tolist() == want


def test_split_parts_merge_to_dense_prefix():
    n, page = 100, 16                  # ragged last page
    q = rng.standard_normal((3, 4, 8))
    k = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    kmin, kmax = Q.page_meta(k, page)
    sel = Q.topk_pages(Q.page_bound(q, kmin, kmax), 3)
    (a_s, l_s), (a_r, l_r) = Q.split_attn(q, k, v, sel, page, 0.35)
    am, lm = merge(a_s, l_s, a_r, l_r)
    a, l = attn_gqa(q, k, v, 0.35)
    np.testing.assert_allclose(am, a, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lm, l, rtol=1e-13)
    # selected part equals attention over exactly the selected tokens
    idx = Q.token_index(sel[1, 0], page, n)
    a1, _ = attn_gqa(q[1:2, 0:2], k[idx][:, 0:1], v[idx][:, 0:1], 0.35)
    np.testing.assert_allclose(a_s[1, 0:2], a1[0], rtol=1e-13)


def test_union_size_brute_force():
    sel = rng.integers(0, 50, size=(8, 3, 6))
    act = np.array([1, 0, 1, 1, 0, 0, 1, 0], dtype=bool)
    u = Q.union_size(sel, act)
    for g in range(3):
        s = set()
        for t in range(8):
            if act[t]:
                s |= set(sel[t, g].tolist())
        assert u[g] == len(s)
    assert Q.union_size(sel, np.zeros(8, bool)).tolist() == [0, 0, 0]
