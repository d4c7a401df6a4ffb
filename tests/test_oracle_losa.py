"""Pins for LoSA's per-step variant (oracle.controller.losa_block) and the
per-query-head selection granularity (oracle.quest.page_bound_heads,
union_size_heads)."""

import numpy as np

import workloads as W
from oracle import controller as C
from oracle import quest as Q
from oracle.attention import attn_gqa, merge


def _small(n_prefix=200, n_steps=4, m_override=None, hq=4, hkv=2, d=16, density=0.25):
    cfg = W.SPARSE.with_(n_prefix=n_prefix, n_block=8, n_steps=n_steps, n_q_heads=hq,
                         n_kv_heads=hkv, head_dim=d, density=density)
    kp, vp = W.prefix_kv(cfg)
    steps = W.sparse_steps(cfg, m_override=m_override)
    conv = [dict(q=W.values(s["q"], cfg.dtype), k=W.values(s["k"], cfg.dtype),
                 v=W.values(s["v"], cfg.dtype)) for s in steps]
    return cfg, W.values(kp, cfg.dtype), W.values(vp, cfg.dtype), conv


def test_losa_hand_example_selects_with_the_current_query():
    # 4 pages of 2 identical keys; key of page p = 5 e_p, value of page p = p.
    # Token 0's query points at page 0 at step 0 and at page 2 at step 1, so
    # with k = 1 it must attend to page 2 alone at step 1: its output is the
    # value of page 2 exactly (equal scores within a page). Tokens 1-3 do not
    # change (MSE 0): nearest-rank cutoff of 4 tokens at 25% is the smallest
    # MSE, 0, so only token 0 is active.
    d, page = 4, 2
    k_p = np.zeros((8, 1, d))
    v_p = np.zeros((8, 1, d))
    for p in range(4):
        k_p[2 * p:2 * p + 2, 0, p] = 5.0
        v_p[2 * p:2 * p + 2, 0, :] = float(p)
    q0 = np.zeros((4, 1, d))
    q0[:, 0, 0] = 1.0
    q1 = q0.copy()
    q1[0, 0, :] = [0.0, 0.0, 1.0, 0.0]
    blk = np.zeros((4, 1, d))
    steps = [dict(q=q0, k=blk, v=blk), dict(q=q1, k=blk, v=blk)]
    recs = C.losa_block(steps, k_p, v_p, 1.0, k_pages=1, page=page)
    assert recs[0]["active"].all()
    assert recs[1]["active"].tolist() == [True, False, False, False]
    assert recs[0]["sel"][:, 0, 0].tolist() == [0, 0, 0, 0]
    assert recs[1]["sel"][:, 0, 0].tolist() == [2, 0, 0, 0]
    np.testing.assert_array_equal(recs[1]["a_out"][0, 0], [2.0] * d)
    assert recs[1]["l_out"][0, 0] == np.log(2.0) + 5.0           # two keys of score 5
    # stable tokens keep the dense step-0 result bit for bit
    np.testing.assert_array_equal(recs[1]["a_out"][1:], recs[0]["a_out"][1:])
    assert recs[1]["union"].tolist() == [1] and recs[1]["union_all"].tolist() == [2]


def test_losa_first_step_is_dense():
    cfg, kp, vp, steps = _small()
    recs = C.losa_block(steps, kp, vp, cfg.scale, k_pages=3, page=16)
    a, l = attn_gqa(steps[0]["q"], kp, vp, cfg.scale)
    np.testing.assert_array_equal(recs[0]["a_out"], a)
    np.testing.assert_array_equal(recs[0]["l_out"], l)


def test_losa_every_page_selected_is_dense_for_active_rows():
    cfg, kp, vp, steps = _small(n_prefix=100, m_override=[None, 3, 8, 1])
    n_pages = Q.n_pages(100, 16)
    recs = C.losa_block(steps, kp, vp, cfg.scale, k_pages=n_pages, page=16)
    for s in range(1, len(steps)):
        a, l = attn_gqa(steps[s]["q"], kp, vp, cfg.scale)
        act = recs[s]["active"]
        assert act.any()
        np.testing.assert_allclose(recs[s]["a_out"][act], a[act], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(recs[s]["l_out"][act], l[act], rtol=1e-12)


def test_losa_active_part_and_the_left_out_pages_merge_to_dense():
    """The pages LoSA drops are exactly FlashBlock's residual: merging the
    active rows' sparse pair with attention over the complement of their
    selection gives dense attention."""
    cfg, kp, vp, steps = _small(m_override=[None, 2, 5, 1])
    recs = C.losa_block(steps, kp, vp, cfg.scale, k_pages=4, page=16)
    for s in range(1, len(steps)):
        rows = np.nonzero(recs[s]["active"])[0]
        q = steps[s]["q"][rows]
        _, (ar, lr) = Q.split_attn(q, kp, vp, recs[s]["sel"][rows], 16, cfg.scale)
        am, lm = merge(recs[s]["a_out"][rows], recs[s]["l_out"][rows], ar, lr)
        a, l = attn_gqa(q, kp, vp, cfg.scale)
        np.testing.assert_allclose(am, a, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(lm, l, rtol=1e-12)


def test_losa_stable_rows_reuse_and_unions():
    cfg, kp, vp, steps = _small(m_override=[None, 2, 0, 3])
    recs = C.losa_block(steps, kp, vp, cfg.scale, k_pages=3, page=16)
    for s in range(1, len(steps)):
        stable = ~recs[s]["active"]
        np.testing.assert_array_equal(recs[s]["a_out"][stable], recs[s - 1]["a_out"][stable])
        sel, act = recs[s]["sel"], recs[s]["active"]
        for g in range(cfg.n_kv_heads):
            u = set()
            for t in range(sel.shape[0]):
                if act[t]:
                    u |= set(int(x) for x in sel[t, g])
            assert recs[s]["union"][g] == len(u)
            assert len(u) <= recs[s]["union_all"][g] <= min(8 * 3, Q.n_pages(200, 16))


def test_per_head_bound_is_a_bound_and_its_group_max_is_the_group_bound():
    cfg, kp, vp, steps = _small(n_prefix=130, hq=8, hkv=2, d=8)
    q = steps[1]["q"]
    kmin, kmax = Q.page_meta(kp, 16)
    bh = Q.page_bound_heads(q, kmin, kmax)
    bg = Q.page_bound(q, kmin, kmax)
    G = 4
    for g in range(2):
        np.testing.assert_array_equal(bh[:, g * G:(g + 1) * G].max(axis=1), bg[:, g])
    for h in range(8):
        g = h // G
        for p in range(Q.n_pages(130, 16)):
            scores = q[:, h, :] @ kp[p * 16:(p + 1) * 16, g, :].T       # [B, tokens]
            assert (scores.max(axis=1) <= bh[:, h, p] + 1e-12).all()


def test_union_size_heads_brute_force():
    rng = np.random.default_rng(5)
    sel = np.sort(rng.integers(0, 40, size=(6, 8, 5)), axis=2)
    active = np.array([1, 0, 1, 1, 0, 0], dtype=bool)
    got = Q.union_size_heads(sel, active, 2)
    for g in range(2):
        u = {int(x) for t in range(6) if active[t] for h in range(4 * g, 4 * g + 4)
             for x in sel[t, h]}
        assert got[g] == len(u)
    assert Q.union_size_heads(sel, np.zeros(6, bool), 2).tolist() == [0, 0]


def test_single_page_selection_per_head_is_the_argmax():
    # k = 1 per query head: the page holding the head's best key upper bound
    cfg, kp, vp, steps = _small(n_prefix=64, hq=2, hkv=1, d=4)
    q = steps[0]["q"]
    kmin, kmax = Q.page_meta(kp, 16)
    bh = Q.page_bound_heads(q, kmin, kmax)
    sel = Q.topk_pages(bh, 1)
    for t in range(q.shape[0]):
        for h in range(2):
            best = max(range(4), key=lambda p: (bh[t, h, p], -p))
            assert sel[t, h, 0] == best
