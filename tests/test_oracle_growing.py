"""Pins for the outer loop over blocks (oracle.growing) and the
count-since-refresh reading of M (oracle.controller.text_block).
"""

import json
import os

import numpy as np

import workloads as W
from oracle import controller as C
from oracle import growing as G
from oracle import quest
from oracle.attention import attn_gqa

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------- count since refresh

def _fixture_steps(ids):
    cfg = W.TINY.with_(n_prefix=32, n_block=len(ids[0]), n_steps=len(ids))
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    for s, st in enumerate(steps):
        st["ids"] = np.array(ids[s], dtype=np.int32)
    return cfg, kp, vp, steps


def test_since_refresh_hand_fixture():
    g = load("text_controller_since_refresh.json")
    cfg, kp, vp, steps = _fixture_steps(g["ids"])
    per = C.text_block(steps, kp, vp, cfg.scale, tau=g["tau"], with_dense=False)
    assert [r["m_count"] for r in per] == g["per_step"]["m_count"]
    assert [r["decision"] for r in per] == g["per_step"]["decision"]
    since = C.text_block(steps, kp, vp, cfg.scale, tau=g["tau"], with_dense=False,
                         since_refresh=True)
    assert [r["m_count"] for r in since] == g["since_refresh"]["m_count"]
    assert [r["decision"] for r in since] == g["since_refresh"]["decision"]
    assert [r["stale"].tolist() for r in since] == g["since_refresh"]["stale"]


def test_since_refresh_brute_force():
    cfg = W.TINY.with_(n_prefix=40, n_block=8, n_steps=14, m_dist="binomial", m_p=0.2)
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg, variant=3)
    for tau in (1, 2, 3, 5):
        recs = C.text_block(steps, kp, vp, cfg.scale, tau=tau, with_dense=False,
                            since_refresh=True)
        ref = [int(x) for x in steps[0]["ids"]]
        for s in range(1, len(steps)):
            cur = [int(x) for x in steps[s]["ids"]]
            m = sum(1 for i in range(len(cur)) if cur[i] != ref[i])
            assert recs[s]["m_count"] == m
            assert recs[s]["decision"] == (C.REUSE if m < tau else C.RECOMPUTE)
            if m >= tau:
                ref = cur
        # on reuse steps M is the number of stale rows
        for r in recs[1:]:
            if r["decision"] == C.REUSE:
                assert int(r["stale"].sum()) == r["m_count"]


def test_since_refresh_equals_per_step_when_every_step_computes():
    cfg = W.TINY.with_(n_prefix=40, n_block=6, n_steps=9)
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg, variant=5)
    a = C.text_block(steps, kp, vp, cfg.scale, tau=0, with_dense=False)
    b = C.text_block(steps, kp, vp, cfg.scale, tau=0, with_dense=False, since_refresh=True)
    assert [r["m_count"] for r in a] == [r["m_count"] for r in b]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x["a_full"], y["a_full"])


# ---------------------------------------------------------------- growing cache

def _whole_sequence_blocks(cfg, n_blocks):
    """Blocks whose last-step K/V are the continuation of one long sequence.

    The prefix generator seeds each 64k-token chunk alone, so a shorter
    prefix is the leading part of a longer one: drawing n0 + n_blocks * B
    tokens once gives a sequence whose slices are what the grown cache must
    hold after each block.
    """
    n0, b = cfg.n_prefix, cfg.n_block
    k_all, v_all = W.prefix_kv(cfg, n_tok=n0 + n_blocks * b)
    blocks = []
    for j in range(n_blocks):
        steps = W.text_steps(cfg, block=j)
        lo = n0 + j * b
        steps[-1] = dict(steps[-1], k=k_all[lo:lo + b].copy(), v=v_all[lo:lo + b].copy())
        blocks.append(steps)
    return k_all, v_all, blocks


def test_growing_cache_is_the_whole_sequence():
    cfg = W.TINY.with_(n_prefix=50, n_block=4, n_steps=3, n_kv_heads=2)
    nb = 4
    k_all, v_all, blocks = _whole_sequence_blocks(cfg, nb)
    kp = W.values(k_all[:cfg.n_prefix], cfg.dtype)
    vp = W.values(v_all[:cfg.n_prefix], cfg.dtype)
    blocks_v = [[dict(st, q=W.values(st["q"], cfg.dtype), k=W.values(st["k"], cfg.dtype),
                      v=W.values(st["v"], cfg.dtype)) for st in steps] for steps in blocks]
    out, (kc, vc) = G.run_blocks(blocks_v, kp, vp, C.text_block, scale=cfg.scale, tau=0,
                                 with_dense=False)
    np.testing.assert_array_equal(kc, W.values(k_all, cfg.dtype))
    np.testing.assert_array_equal(vc, W.values(v_all, cfg.dtype))
    for j, blk in enumerate(out):
        n_j = cfg.n_prefix + j * cfg.n_block
        assert blk["n_prefix"] == n_j
        last = blk["recs"][-1]
        # the last step of block j attends over the first n_j + B tokens of
        # the sequence: one attention over a slice, no merge
        q = blocks_v[j][-1]["q"]
        a, l = attn_gqa(q, W.values(k_all[:n_j + cfg.n_block], cfg.dtype),
                        W.values(v_all[:n_j + cfg.n_block], cfg.dtype), cfg.scale)
        np.testing.assert_allclose(last["a_full"], a, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(last["l_full"], l, rtol=1e-12)
        # every step's block-external pair is attention over the first n_j tokens
        for r, st in zip(blk["recs"], blocks_v[j]):
            a, l = attn_gqa(st["q"], W.values(k_all[:n_j], cfg.dtype),
                            W.values(v_all[:n_j], cfg.dtype), cfg.scale)
            np.testing.assert_array_equal(r["a_out"], a)
            np.testing.assert_array_equal(r["l_out"], l)


def test_growing_run_appends_after_each_block_in_order():
    cfg = W.TINY.with_(n_prefix=6, n_block=3, n_steps=2, n_kv_heads=1, n_q_heads=1, head_dim=4)
    kp = np.zeros((6, 1, 4))
    vp = np.zeros((6, 1, 4))
    blocks = []
    for j in range(3):
        steps = []
        for s in range(2):
            mark = np.full((3, 1, 4), 10.0 * j + s)
            steps.append(dict(q=np.zeros((3, 1, 4)), k=mark, v=mark + 0.5,
                              ids=np.arange(3, dtype=np.int32)))
        blocks.append(steps)
    seen = []

    def probe(steps, k_c, v_c, **kw):
        seen.append(np.asarray(k_c)[:, 0, 0].tolist())
        return []

    _, (kc, vc) = G.run_blocks(blocks, kp, vp, probe)
    assert seen == [[0.0] * 6, [0.0] * 6 + [1.0] * 3, [0.0] * 6 + [1.0] * 3 + [11.0] * 3]
    assert kc[:, 0, 0].tolist() == [0.0] * 6 + [1.0] * 3 + [11.0] * 3 + [21.0] * 3
    assert vc[:, 0, 0].tolist() == [0.0] * 6 + [1.5] * 3 + [11.5] * 3 + [21.5] * 3


def test_page_meta_of_full_pages_survives_growth():
    """The incremental update's premise: a page whose tokens all lie inside
    the old cache keeps its min/max when tokens are appended; only the old
    partial last page and the new pages change."""
    cfg = W.SPARSE.with_(n_prefix=200, n_kv_heads=2, head_dim=8)
    k_all, _ = W.prefix_kv(cfg, n_tok=200)
    k = W.values(k_all, cfg.dtype)
    page = 16
    for n1, n2 in ((37, 38), (37, 64), (48, 49), (48, 200), (1, 17)):
        m1, x1 = quest.page_meta(k[:n1], page)
        m2, x2 = quest.page_meta(k[:n2], page)
        full = n1 // page
        np.testing.assert_array_equal(m1[:, :full], m2[:, :full])
        np.testing.assert_array_equal(x1[:, :full], x2[:, :full])
        if n1 % page:
            # the partial page widens (never narrows) as tokens arrive
            assert (m2[:, full] <= m1[:, full]).all() and (x2[:, full] >= x1[:, full]).all()


def test_sparse_blocks_refresh_over_the_grown_cache_is_dense():
    cfg = W.SPARSE.with_(n_prefix=80, n_block=4, n_steps=2, n_q_heads=4, n_kv_heads=2,
                         head_dim=16)
    nb = 3
    k_all, v_all, blocks = _whole_sequence_blocks(cfg, nb)
    conv = [[dict(st, q=W.values(st["q"], cfg.dtype), k=W.values(st["k"], cfg.dtype),
                  v=W.values(st["v"], cfg.dtype)) for st in steps] for steps in blocks]
    kp = W.values(k_all[:cfg.n_prefix], cfg.dtype)
    vp = W.values(v_all[:cfg.n_prefix], cfg.dtype)
    out, _ = G.run_blocks(conv, kp, vp, C.sparse_block, scale=cfg.scale, k_pages=2, page=16)
    for j, blk in enumerate(out):
        n_j = cfg.n_prefix + j * cfg.n_block
        r0 = blk["recs"][0]
        a, l = attn_gqa(conv[j][0]["q"], W.values(k_all[:n_j], cfg.dtype),
                        W.values(v_all[:n_j], cfg.dtype), cfg.scale)
        np.testing.assert_allclose(r0["a_out"], a, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(r0["l_out"], l, rtol=1e-12)
        assert r0["sel"].max() < -(-n_j // 16)
