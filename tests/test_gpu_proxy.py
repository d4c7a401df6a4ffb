"""GPU parity of the singular-proxy identifier (fb_proxy_decide) against
oracle.spa: proxies and cache within the rounding bound of a float64 dot
product of d_model exact products, similarities within SIM_ATOL, and the
selected token ids and masks exactly wherever the oracle's similarities leave
a margin at the selection boundary (asserted per step)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import spa as OS
from _helpers import SIM_ATOL, cpu, sim_margin_ok

pytestmark = pytest.mark.gpu


def check_proxy(name, got, x, f, want):
    """|p_gpu - p_oracle| <= 2 d_model 2^-53 (|x| |F|) per entry: both sums of
    the same exact products, each within d_model 2^-53 sum |x F| of the exact
    value whatever its order."""
    x = np.asarray(x, dtype=np.float64)
    f = np.asarray(f, dtype=np.float64)
    bound = 2 * x.shape[1] * 2.0 ** -53 * (np.abs(x) @ np.abs(f))
    err = np.abs(np.asarray(got) - want)
    assert np.all(err <= bound), "%s: proxy err %.3g (bound %.3g)" % (
        name, float(err.max()), float(bound[err > bound].min()))


def check_step(tag, idn, x, f, rec, k, cache_src):
    """One step's outputs against the oracle record; cache_src: the GPU
    cache rows are the GPU's own proxies of the steps they were taken at."""
    if rec["sim"] is not None:
        assert sim_margin_ok(rec["sim"], k), tag + ": similarities too close at the boundary"
    check_proxy(tag + " proxy", cpu(idn.proxy), x, f, rec["proxy"])
    assert np.array_equal(cpu(idn.mask).astype(bool), rec["mask"]), tag
    if rec["sim"] is not None:
        assert np.max(np.abs(cpu(idn.sim) - rec["sim"])) <= SIM_ATOL, tag
        if k > 0:
            assert np.array_equal(cpu(idn.selected)[:k], rec["selected"]), tag
    cache = cpu(idn.cache)
    for t in range(cache.shape[0]):
        assert np.array_equal(cache[t], cache_src[t]), (tag, t)


def _dev(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


class Ident:
    """Device buffers of one identifier run."""

    def __init__(self, fb, n, d, r, n_select):
        self.fb, self.n, self.r, self.n_select = fb, n, r, n_select
        f64 = dict(device="cuda", dtype=torch.float64)
        self.cache = torch.full((n, r), 3.0, **f64)
        self.sim = torch.full((n,), 9.0, **f64)
        self.proxy = torch.empty(n, r, **f64)
        self.mask = torch.full((n,), 7, device="cuda", dtype=torch.uint8)
        self.selected = torch.full((max(n_select, 1),), -1, device="cuda", dtype=torch.int32)
        self.d = d

    def step(self, x, f, init, with_proxy=True):
        fb = self.fb
        a = fb.proxy_args(x, f, self.cache, self.mask, self.selected, self.n_select, init,
                          sim=self.sim, proxy=self.proxy if with_proxy else None)
        ws = torch.empty(max(fb.fb_proxy_decide_workspace(a), 16), dtype=torch.uint8, device="cuda")
        a.ws, a.ws_bytes = ws.data_ptr(), ws.numel()
        fb.fb_proxy_decide(a)
        torch.cuda.synchronize()


CASES = [
    # name, n_tok, d_model, rank, n_select, dtype
    ("ragged_r32", 100, 1300, 32, 25, "bf16"),
    ("r64_exact_tiles", 64, 1024, 64, 16, "bf16"),
    ("r96", 70, 700, 96, 7, "bf16"),
    ("r128", 96, 2048, 128, 24, "bf16"),
    ("f32_r64", 50, 600, 64, 13, "f32"),
    ("select_none", 40, 512, 32, 0, "bf16"),
    ("select_all", 40, 512, 32, 40, "bf16"),
    # one token (recomputed or not); 65 tokens (a second selection
    # workgroup holding one token) over a width shorter than one block
    ("one_token", 1, 256, 32, 1, "bf16"),
    ("one_token_none", 1, 256, 32, 0, "bf16"),
    ("t65_d100", 65, 100, 64, 30, "bf16"),
    ("t65_f32_r96", 65, 100, 96, 64, "f32"),
    # the rank-counting selection at its largest size (128 workgroups), and
    # the radix top-k + scatter just beyond it
    ("select_rank_8192", 8192, 256, 32, 2000, "bf16"),
    ("select_radix_8200", 8200, 256, 32, 2050, "bf16"),
]


@pytest.mark.parametrize("name,n,d,r,k,dt", CASES, ids=[c[0] for c in CASES])
def test_identifier_matches_oracle(fb, name, n, d, r, k, dt):
    cfg = W.SPA.with_(n_tok=n, d_model=d, rank=r, n_steps=3, cfg_id=6 if dt == "bf16" else 16)
    fbits = W.spa_factor(cfg)
    steps = W.spa_steps(cfg)
    if dt == "f32":
        fbits = W.values(fbits, "bf16").astype(np.float32) * np.float32(1.0 + 2 ** -12)
        steps = [W.values(x, "bf16").astype(np.float32) * np.float32(1.0 - 2 ** -13) for x in steps]
    fv = W.values(fbits, dt) if dt == "bf16" else fbits
    xs = [W.values(x, dt) if dt == "bf16" else x for x in steps]
    recs = OS.spa_run(xs, fv, k)
    f_d = _dev(fbits, dt)
    idn = Ident(fb, n, d, r, k)
    held = np.zeros((n, r))                  # the GPU's proxies at each token's last recompute
    for s, (x, rec) in enumerate(zip(steps, recs)):
        idn.step(_dev(x, dt), f_d, init=(s == 0))
        p = cpu(idn.proxy)
        held[rec["mask"]] = p[rec["mask"]]
        check_step("%s step %d" % (name, s), idn, xs[s], fv, rec, k, held)


def test_identifier_exact_on_small_integers(fb):
    # integer states and factor: every partial sum is an exact integer, so
    # the proxies equal the oracle's bit for bit in any order
    n, d, r = 40, 700, 32
    rng = np.random.default_rng(5)
    x = rng.integers(-8, 9, size=(n, d)).astype(np.float32)
    f = rng.integers(-8, 9, size=(d, r)).astype(np.float32)
    idn = Ident(fb, n, d, r, 0)
    idn.step(_dev(W.bf16_bits(x), "bf16"), _dev(W.bf16_bits(f), "bf16"), init=True)
    assert np.array_equal(cpu(idn.proxy), OS.proxy(x, f))
    assert np.array_equal(cpu(idn.cache), OS.proxy(x, f))


@pytest.mark.parametrize("n,k", [(50, 9), (300, 130), (8200, 3000)])
def test_identifier_ties_go_to_lower_ids(fb, n, k):
    # every token identical and its cache identical: every similarity is 1
    # (one workgroup, ties across several, and the radix top-k)
    d, r = 512, 32
    rng = np.random.default_rng(0)
    row = W.bf16_bits(rng.standard_normal((1, d)).astype(np.float32))
    x = np.repeat(row, n, axis=0)
    f = W.spa_factor(W.SPA.with_(d_model=d, rank=r))
    idn = Ident(fb, n, d, r, k)
    idn.step(_dev(x, "bf16"), _dev(f, "bf16"), init=True)
    idn.step(_dev(x, "bf16"), _dev(f, "bf16"), init=False, with_proxy=False)
    assert (cpu(idn.sim) == 1.0).all()
    assert cpu(idn.selected)[:k].tolist() == list(range(k))
    assert cpu(idn.mask).astype(bool).tolist() == [t < k for t in range(n)]


def test_identifier_full_size(fb):
    """1024 tokens of width 4096, rank 128, a quarter recomputed per step --
    the size the benchmark times."""
    cfg = W.SPA.with_(n_steps=3)
    f = W.spa_factor(cfg)
    steps = W.spa_steps(cfg)
    xs = [W.values(x, "bf16") for x in steps]
    fv = W.values(f, "bf16")
    recs = OS.spa_run(xs, fv, cfg.n_select)
    idn = Ident(fb, cfg.n_tok, cfg.d_model, cfg.rank, cfg.n_select)
    f_d = _dev(f, "bf16")
    held = np.zeros((cfg.n_tok, cfg.rank))
    for s, (x, rec) in enumerate(zip(steps, recs)):
        idn.step(_dev(x, "bf16"), f_d, init=(s == 0))
        p = cpu(idn.proxy)
        held[rec["mask"]] = p[rec["mask"]]
        check_step("full step %d" % s, idn, xs[s], fv, rec, cfg.n_select, held)


def test_layer_stack_with_depth_budgets(fb):
    """A stack of layers, each with its own value-projection factor and
    hidden-state walk, recomputing the per-layer counts of fb_layer_budgets:
    every layer's selection and cache bit for bit."""
    from oracle import budget as OB
    n_layers, n, d, r = 4, 96, 640, 32
    ratios, counts = fb.fb_layer_budgets(n_layers, n, 0.16, 0.04, 1.5, 1.0, 0.75)
    assert counts == OB.layer_counts(n, OB.layer_ratios(n_layers, 0.16, 0.04, 1.5, 1.0, 0.75)).tolist()
    for layer in range(n_layers):
        cfg = W.SPA.with_(n_tok=n, d_model=d, rank=r, n_steps=3)
        f = W.spa_factor(cfg, variant=layer)
        steps = W.spa_steps(cfg, variant=layer)
        xs, fv = [W.values(x, "bf16") for x in steps], W.values(f, "bf16")
        recs = OS.spa_run(xs, fv, counts[layer])
        idn = Ident(fb, n, d, r, counts[layer])
        f_d = _dev(f, "bf16")
        held = np.zeros((n, r))
        for s, (x, rec) in enumerate(zip(steps, recs)):
            idn.step(_dev(x, "bf16"), f_d, init=(s == 0))
            p = cpu(idn.proxy)
            held[rec["mask"]] = p[rec["mask"]]
            check_step("layer %d step %d" % (layer, s), idn, xs[s], fv, rec, counts[layer], held)
