"""Pins for the singular-proxy identifier (oracle.spa) and its synthetic
value projection (workloads.spa_factor / spa_projection)."""

import numpy as np

import workloads as W
from oracle import spa as S


def _cos(a, b):
    return np.sum(a * b, axis=1) / (np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1))


def test_projection_has_the_stated_svd():
    cfg = W.SPA.with_(d_model=48)
    u, sig, v = W.spa_projection(cfg)
    w = u @ np.diag(sig) @ v.T
    s = np.linalg.svd(w, compute_uv=False)
    np.testing.assert_allclose(s, sig, rtol=1e-12)
    np.testing.assert_allclose(sig, 1.0 / np.sqrt(np.arange(1, 49)), rtol=1e-15)
    np.testing.assert_allclose(u.T @ u, np.eye(48), atol=1e-13)
    np.testing.assert_allclose(v.T @ v, np.eye(48), atol=1e-13)


def test_factor_has_orthogonal_columns_scaled_by_the_spectrum():
    cfg = W.SPA.with_(d_model=256, rank=16)
    f = W.values(W.spa_factor(cfg), "bf16").astype(np.float64)
    g = f.T @ f                                   # diag(sigma^2) up to bf16 rounding
    np.testing.assert_allclose(np.diag(g), W.spectrum(16) ** 2, rtol=2e-2)
    off = g - np.diag(np.diag(g))
    assert np.abs(off).max() < 2e-2 * g.max()


def test_proxy_cosine_is_the_rank_r_value_state_cosine():
    """V orthonormal: cos(x U_r S_r, y U_r S_r) = cos(x W_r, y W_r), and with
    r = D the proxy cosine is the cosine of the value states x W."""
    cfg = W.SPA.with_(d_model=40, n_tok=12)
    u, sig, v = W.spa_projection(cfg)
    rng = np.random.default_rng(1)
    x, y = rng.standard_normal((12, 40)), rng.standard_normal((12, 40))
    for r in (5, 40):
        f = u[:, :r] * sig[:r]
        w_r = f @ v[:, :r].T
        kp = S.proxy_key(S.proxy(x, f), S.proxy(y, f))
        c = _cos(x @ w_r, y @ w_r)
        np.testing.assert_allclose(kp, np.sign(c) * c * c, rtol=1e-12, atol=1e-15)
    w = u @ np.diag(sig) @ v.T
    c = _cos(x @ w, y @ w)
    kp = S.proxy_key(S.proxy(x, u * sig), S.proxy(y, u * sig))
    np.testing.assert_allclose(kp, np.sign(c) * c * c, rtol=1e-12, atol=1e-15)


def test_proxy_matches_matmul_and_is_exact_on_integers():
    rng = np.random.default_rng(2)
    x = W.values(W.bf16_bits(rng.standard_normal((9, 1100)).astype(np.float32)), "bf16")
    f = W.values(W.bf16_bits(rng.standard_normal((1100, 24)).astype(np.float32)), "bf16")
    np.testing.assert_allclose(S.proxy(x, f), x.astype(np.float64) @ f.astype(np.float64),
                               rtol=1e-12, atol=1e-12)
    xi = rng.integers(-50, 50, size=(5, 1300)).astype(np.float64)
    fi = rng.integers(-50, 50, size=(1300, 7)).astype(np.float64)
    np.testing.assert_array_equal(S.proxy(xi, fi), xi @ fi)


def test_proxy_sums_in_blocks_of_128():
    # x = 2^53 at c = 0 and 1 at c = 128, 129: block 0 sums to 2^53, block 1
    # to 2, total 2^53 + 2 (exact); one running sum over c would round each
    # +1 away and give 2^53.
    d = 2 * S.PROXY_BLOCK
    x = np.zeros((1, d))
    x[0, 0] = 2.0 ** 53
    x[0, S.PROXY_BLOCK] = x[0, S.PROXY_BLOCK + 1] = 1.0
    f = np.ones((d, 1))
    assert S.proxy(x, f)[0, 0] == 2.0 ** 53 + 2.0
    run = 0.0
    for c in range(d):
        run = run + x[0, c]
    assert run == 2.0 ** 53


def test_key_hand_values_and_conventions():
    p = np.array([[1.0, 0.0], [1.0, 1.0], [2.0, 0.0], [0.0, 0.0], [0.0, 0.0], [3.0, 4.0]])
    c = np.array([[1.0, 1.0], [1.0, 1.0], [-3.0, 0.0], [0.0, 0.0], [1.0, 0.0], [3.0, 4.0]])
    k = S.proxy_key(p, c)
    assert k[0] == 0.5                     # cos = 1/sqrt(2)
    assert k[1] == 1.0 and k[5] == 1.0     # identical proxies: exactly 1
    assert k[2] == -1.0                    # opposite
    assert k[3] == 1.0 and k[4] == 0.0     # both zero / one zero
    # orthogonal: 0 (not -0)
    z = S.proxy_key(np.array([[1.0, 0.0]]), np.array([[0.0, -1.0]]))
    assert z[0] == 0.0 and not np.signbit(z[0])


def test_key_orders_like_the_cosine():
    rng = np.random.default_rng(3)
    p, c = rng.standard_normal((300, 16)), rng.standard_normal((300, 16))
    k = S.proxy_key(p, c)
    cos = _cos(p, c)
    np.testing.assert_array_equal(np.argsort(k, kind="stable"), np.argsort(cos, kind="stable"))


def test_select_lowest_brute_force_and_ties():
    key = np.array([0.5, 0.2, 0.9, 0.2, -0.1, 0.5, 0.2])
    assert S.select_lowest(key, 3).tolist() == [1, 3, 4]
    assert S.select_lowest(key, 4).tolist() == [1, 3, 4, 6]
    assert S.select_lowest(key, 0).tolist() == []
    rng = np.random.default_rng(4)
    key = rng.integers(0, 6, size=50).astype(np.float64)
    for k in (1, 7, 25, 50):
        brute = sorted(sorted(range(50), key=lambda t: (key[t], t))[:k])
        assert S.select_lowest(key, k).tolist() == brute


def test_run_caches_at_recompute_and_still_tokens_are_exactly_similar():
    cfg = W.SPA.with_(n_tok=40, d_model=600, rank=8, n_steps=4)
    f = W.values(W.spa_factor(cfg), "bf16")
    steps = [W.values(x, "bf16") for x in W.spa_steps(cfg)]
    steps[2] = steps[1].copy()                    # no token moves between steps 1 and 2
    recs = S.spa_run(steps, f, n_select=10)
    assert recs[0]["mask"].all() and recs[0]["key"] is None
    np.testing.assert_array_equal(recs[0]["cache"], S.proxy(steps[0], f))
    for s in range(1, 4):
        r = recs[s]
        assert r["selected"].size == 10 and r["mask"].sum() == 10
        prev = recs[s - 1]["cache"]
        np.testing.assert_array_equal(r["cache"][r["mask"]], r["proxy"][r["mask"]])
        np.testing.assert_array_equal(r["cache"][~r["mask"]], prev[~r["mask"]])
        # every selected token is at most as similar as every other one
        assert r["key"][r["mask"]].max() <= r["key"][~r["mask"]].min()
    # tokens recomputed at step 1 have key exactly 1 at step 2 (same state)
    assert (recs[2]["key"][recs[1]["mask"]] == 1.0).all()


def test_drift_scales_order_the_selection():
    # the walk's per-token drift decides who is least similar: the tokens
    # picked at step 1 drift more than the median token
    cfg = W.SPA.with_(n_tok=64, d_model=512, rank=16, n_steps=2)
    f = W.values(W.spa_factor(cfg), "bf16")
    steps = [W.values(x, "bf16") for x in W.spa_steps(cfg)]
    recs = S.spa_run(steps, f, n_select=8)
    move = np.linalg.norm(steps[1] - steps[0], axis=1)
    assert np.median(move[recs[1]["mask"]]) > np.median(move)
