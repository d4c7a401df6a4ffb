"""Pins for oracle.controller: the count, cosine and active-set decisions and
the per-step text / video / sparse FlashBlock paths.
"""

import json
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import controller as C
from oracle.attention import attn_gqa, dense_step, merge

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(99)


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ count

def test_count_hand_fixture():
    g = load("text_controller.json")
    ids = g["ids"]
    for s in range(1, len(ids)):
        assert C.count_updated(ids[s - 1], ids[s]) == g["m_count"][s]
        assert (C.REUSE if C.text_reuse(g["m_count"][s], g["tau"]) else C.RECOMPUTE) == g["decision"][s]


def test_count_brute_force_and_generator_draws():
    cfg = W.TINY.with_(n_block=16, n_steps=12, m_dist="binomial")
    steps = W.text_steps(cfg)
    for s in range(1, len(steps)):
        a, b = steps[s - 1]["ids"], steps[s]["ids"]
        brute = sum(1 for i in range(len(a)) if int(a[i]) != int(b[i]))
        assert C.count_updated(a, b) == brute == steps[s]["m_drawn"]


def test_tau_boundary_is_strict():
    assert C.text_reuse(1, 2) and not C.text_reuse(2, 2) and not C.text_reuse(3, 2)
    assert not C.text_reuse(0, 0)


# ------------------------------------------------------------------ cosine

def test_cosine_hand_values():
    a = np.zeros((1, 3, 2))
    b = np.zeros((1, 3, 2))
    a[0, 0] = [1, 0]; b[0, 0] = [1, 1]          # 1/sqrt(2)
    a[0, 1] = [2, 0]; b[0, 1] = [-3, 0]         # -1
    a[0, 2] = [0, 0]; b[0, 2] = [0, 0]          # both zero -> 1
    sim = C.head_cosine(a, b)
    assert sim[0] == pytest.approx(1 / math.sqrt(2), rel=1e-15)
    assert sim[1] == -1.0
    assert sim[2] == 1.0
    b[0, 2] = [1, 0]
    assert C.head_cosine(a, b)[2] == 0.0


def test_cosine_brute_force_and_scale_invariance():
    a, b = rng.standard_normal((5, 3, 4)), rng.standard_normal((5, 3, 4))
    sim = C.head_cosine(a, b)
    for h in range(3):
        x = [a[i, h, j] for i in range(5) for j in range(4)]
        y = [b[i, h, j] for i in range(5) for j in range(4)]
        dot = sum(p * q for p, q in zip(x, y))
        want = dot / math.sqrt(sum(p * p for p in x)) / math.sqrt(sum(q * q for q in y))
        assert sim[h] == pytest.approx(want, rel=1e-13)
    np.testing.assert_allclose(C.head_cosine(3.0 * a, 0.5 * b), sim, rtol=1e-13)
    assert np.all(C.head_cosine(a, a) <= 1.0)


def test_gamma_boundary_is_strict():
    assert list(C.head_reuse([0.95, 0.9500001, 1.0], 0.95)) == [False, True, True]


# ------------------------------------------------------------- active set

def test_active_set_hand_fixture():
    g = load("active_set_toy.json")
    qp = np.array(g["q_prev"], dtype=np.float64)[:, None, :]
    qc = np.array(g["q_cur"], dtype=np.float64)[:, None, :]
    mse = C.active_mse(qp, qc)
    np.testing.assert_array_equal(mse, g["mse"])
    assert C.percentile_cutoff(mse) == g["cutoff"]
    assert list(C.active_set(mse)) == g["active"]


def test_mse_matches_mean_of_squares_and_zero_when_unchanged():
    a = rng.standard_normal((8, 4, 16))
    b = a.copy()
    b[[1, 5]] += rng.standard_normal((2, 4, 16))
    mse = C.active_mse(a, b)
    np.testing.assert_allclose(mse, ((b - a) ** 2).mean(axis=(1, 2)), rtol=1e-14)
    assert np.all(mse[[0, 2, 3, 4, 6, 7]] == 0.0)
    # pure-python brute force on one token
    want = sum((b[5, h, j] - a[5, h, j]) ** 2 for h in range(4) for j in range(16)) / 64
    assert mse[5] == pytest.approx(want, rel=1e-14)


def test_nearest_rank_agrees_with_linear_percentile_for_b8():
    # For B = 8 (sorted x[0..7]) the nearest-rank cutoff is x[1]; numpy's
    # linear interpolation gives c = x[1] + 0.75 (x[2] - x[1]). If x[2] > x[1]
    # then x[i] > c for every i >= 2 and x[0], x[1] <= c, so both rules select
    # i >= 2 among distinct values; if x[2] == x[1], c == x[1]. Same sets.
    for trial in range(200):
        x = rng.standard_normal(8) ** 2
        if trial % 3 == 0:
            x[rng.choice(8, 3, replace=False)] = 0.0
        act = C.active_set(x, 25)
        lin = x > np.percentile(x, 25)
        assert list(act) == list(lin)
        srt = sorted(x.tolist())
        assert C.percentile_cutoff(x, 25) == srt[1]


# ---------------------------------------------------------------- text path

def _tiny(n_prefix=96, n_block=4, n_steps=7, m_override=None, **kw):
    cfg = W.TINY.with_(n_prefix=n_prefix, n_block=n_block, n_steps=n_steps, **kw)
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg, m_override=m_override)
    return cfg, kp, vp, steps


def test_text_tau_zero_recomputes_and_matches_dense():
    cfg, kp, vp, steps = _tiny()
    recs = C.text_block(steps, kp, vp, cfg.scale, tau=0)
    assert [r["decision"] for r in recs] == [C.INIT] + [C.RECOMPUTE] * (len(steps) - 1)
    for r in recs:
        np.testing.assert_allclose(r["a_full"], r["a_dense"], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(r["l_full"], r["l_dense"], rtol=1e-12)
        assert not r["stale"].any()


def test_text_tau_above_b_always_reuses():
    cfg, kp, vp, steps = _tiny()
    recs = C.text_block(steps, kp, vp, cfg.scale, tau=cfg.n_block + 1)
    assert [r["decision"] for r in recs] == [C.INIT] + [C.REUSE] * (len(steps) - 1)
    for r in recs[1:]:
        assert r["a_out"] is recs[0]["a_out"]


def test_text_fresh_rows_exact_stale_rows_flagged():
    # rows whose token did not change since the last compute step see the
    # same static prefix with the same query, so the cached pair is exact and
    # the merged output equals dense attention; changed rows are stale.
    cfg, kp, vp, steps = _tiny(n_block=6, n_steps=8,
                               m_override=[None, 1, 0, 2, 5, 1, 0, 2])
    recs = C.text_block(steps, kp, vp, cfg.scale, tau=3)
    assert [r["decision"] for r in recs] == [C.INIT, C.REUSE, C.REUSE, C.REUSE,
                                             C.RECOMPUTE, C.REUSE, C.REUSE, C.REUSE]
    assert any(r["decision"] == C.REUSE and r["stale"].any() for r in recs)
    for r in recs:
        fresh = ~r["stale"]
        np.testing.assert_allclose(r["a_full"][fresh], r["a_dense"][fresh], rtol=1e-11, atol=1e-13)
        if r["stale"].any():
            assert not np.allclose(r["a_full"][r["stale"]], r["a_dense"][r["stale"]])


def test_text_controller_follows_hand_fixture():
    g = load("text_controller.json")
    cfg = W.TINY.with_(n_prefix=32, n_block=4, n_steps=len(g["ids"]))
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    for s, st in enumerate(steps):
        st["ids"] = np.array(g["ids"][s], dtype=np.int32)
    recs = C.text_block(steps, kp, vp, cfg.scale, tau=g["tau"], with_dense=False)
    assert [r["decision"] for r in recs] == g["decision"]
    assert [r["m_count"] for r in recs] == g["m_count"]
    assert [r["stale"].tolist() for r in recs] == g["stale"]


def test_text_merge_of_parts():
    cfg, kp, vp, steps = _tiny(n_steps=3)
    recs = C.text_block(steps, kp, vp, cfg.scale, tau=2)
    r = recs[-1]
    ai, li = attn_gqa(steps[-1]["q"], steps[-1]["k"], steps[-1]["v"], cfg.scale)
    np.testing.assert_array_equal(r["a_in"], ai)
    am, lm = merge(r["a_out"], r["l_out"], ai, li)
    np.testing.assert_array_equal(r["a_full"], am)


# --------------------------------------------------------------- video path

def _video(sigmas, n_block=24, n_prefix=40, heads=3, d=8, n_steps=4):
    cfg = W.VIDEO.with_(n_block=n_block, n_prefix=n_prefix, n_q_heads=heads,
                        n_kv_heads=heads, head_dim=d, n_steps=n_steps)
    kp, vp = W.prefix_kv(cfg)
    steps = W.video_steps(cfg, sigmas)
    return cfg, kp, vp, steps


def test_video_zero_noise_reuses_exactly():
    cfg, kp, vp, steps = _video([0.0, 0.0, 0.0])
    recs = C.video_block(steps, kp, vp, cfg.scale, gamma=0.95, with_dense=True)
    assert recs[1]["decisions"] == [C.RECOMPUTE] * 3          # the probe step
    assert np.all(recs[1]["sim"] == 1.0)
    assert recs[2]["decisions"] == [C.REUSE] * 3
    for r in recs:
        np.testing.assert_allclose(r["a_full"], r["a_dense"], rtol=1e-11, atol=1e-13)


def test_video_gamma_extremes():
    sig = [0.5, 0.01, 0.0]
    cfg, kp, vp, steps = _video(sig)
    never = C.video_block(steps, kp, vp, cfg.scale, gamma=1.0)
    assert all(d == C.RECOMPUTE for r in never[1:] for d in r["decisions"])
    always = C.video_block(steps, kp, vp, cfg.scale, gamma=-1.5)
    assert always[1]["decisions"] == [C.RECOMPUTE] * 3
    assert all(d == C.REUSE for r in always[2:] for d in r["decisions"])


def test_video_recomputed_heads_track_similarity():
    sig = [0.8, 0.001, 0.3]
    cfg, kp, vp, steps = _video(sig, n_steps=4)
    recs = C.video_block(steps, kp, vp, cfg.scale, gamma=0.95, with_dense=True)
    for s in (1, 2, 3):
        prev_cache = recs[s - 1]["a_out"]
        for h in range(3):
            if recs[s]["decisions"][h] == C.RECOMPUTE:
                fresh, _ = attn_gqa(steps[s]["q"], kp, vp, cfg.scale, heads=[h])
                want = C.head_cosine(fresh[:, h:h + 1], prev_cache[:, h:h + 1])[0]
                assert recs[s]["sim"][h] == want
                np.testing.assert_array_equal(recs[s]["a_out"][:, h], fresh[:, h])
                assert recs[s]["reuse_next"][h] == (want > 0.95)
                # recomputed heads are exact
                np.testing.assert_allclose(recs[s]["a_full"][:, h], recs[s]["a_dense"][:, h], rtol=1e-11, atol=1e-13)
            else:
                np.testing.assert_array_equal(recs[s]["a_out"][:, h], prev_cache[:, h])


# -------------------------------------------------------------- sparse path

def _sparse(density, n_prefix=256, page=16, n_block=8, n_steps=4, hq=4, hkv=2, d=16):
    cfg = W.SPARSE.with_(n_prefix=n_prefix, page=page, n_block=n_block,
                         n_steps=n_steps, n_q_heads=hq, n_kv_heads=hkv,
                         head_dim=d, density=density)
    kp, vp = W.prefix_kv(cfg)
    steps = W.sparse_steps(cfg)
    return cfg, kp, vp, steps


def test_sparse_refresh_is_dense_and_density_one_is_exact():
    for density in (0.0, 0.25, 1.0):
        cfg, kp, vp, steps = _sparse(density)
        recs = C.sparse_block(steps, kp, vp, cfg.scale, cfg.k_pages, cfg.page, with_dense=True)
        np.testing.assert_allclose(recs[0]["a_full"], recs[0]["a_dense"], rtol=1e-11, atol=1e-13)
        if density == 1.0:
            assert np.all(recs[0]["l_res"] == -np.inf)
            for r in recs:
                np.testing.assert_allclose(r["a_full"], r["a_dense"], rtol=1e-11, atol=1e-13)
        if density == 0.0:
            assert cfg.k_pages == 0


def test_sparse_stable_rows_keep_their_output():
    cfg, kp, vp, steps = _sparse(0.25, n_steps=5)
    recs = C.sparse_block(steps, kp, vp, cfg.scale, cfg.k_pages, cfg.page)
    assert recs[0]["active"].all()
    for s in range(1, len(recs)):
        act = recs[s]["active"]
        changed = np.any(steps[s]["q"] != steps[s - 1]["q"], axis=(1, 2))
        # unchanged tokens have MSE exactly 0 and are never active
        assert not np.any(act & ~changed)
        np.testing.assert_array_equal(recs[s]["a_out"][~act], recs[s - 1]["a_out"][~act])
        u = recs[s]["union"]
        for g in range(cfg.n_kv_heads):
            want = len(set(recs[0]["sel"][act, g].ravel().tolist())) if act.any() else 0
            assert u[g] == want


def test_mse_is_the_exact_mean_rounded_once():
    # Worked by hand. One token, one head, d = 4; q_prev = 0,
    # q_cur = [2^27, 1, 1, 1]: squared differences 2^54, 1, 1, 1. Exact sum
    # 2^54 + 3, mean 2^52 + 0.75, which rounds to 2^52 + 1 (ulp 1 at 2^52).
    # Any float64 running or pairwise sum loses the ones: 2^54 + 1 and
    # 2^54 + 2 both round to 2^54 (ulp 4, ties to even), giving 2^52.
    q_prev = np.zeros((1, 1, 4))
    q_cur = np.array([[[2.0 ** 27, 1.0, 1.0, 1.0]]])
    mse = C.active_mse(q_prev, q_cur)
    assert mse[0] == 2.0 ** 52 + 1.0
    run = 0.0
    for v in (2.0 ** 54, 1.0, 1.0, 1.0):
        run = run + v
    assert run / 4 == 2.0 ** 52
    # a constant shift c changes every value by c: MSE = c^2 exactly
    a = np.round(rng.standard_normal((3, 2, 8)) * 64) / 64     # a + 0.25 exact
    np.testing.assert_array_equal(C.active_mse(a, a + 0.25), np.full(3, 0.0625))


def test_mse_does_not_depend_on_the_order_of_heads_and_dims():
    a = rng.standard_normal((4, 8, 16))
    b = a + rng.standard_normal((4, 8, 16)) * np.array([1.0, 1e-9, 1e7, 3.0])[:, None, None]
    want = C.active_mse(a, b)
    perm = rng.permutation(8 * 16)
    pa = a.reshape(4, -1)[:, perm].reshape(4, 16, 8)
    pb = b.reshape(4, -1)[:, perm].reshape(4, 16, 8)
    np.testing.assert_array_equal(C.active_mse(pa, pb), want)


