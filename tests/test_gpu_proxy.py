"""GPU parity of the singular-proxy identifier (fb_proxy_decide) against
oracle.spa: proxies, keys and cache bit for bit (the float64 arithmetic is
fixed operation by operation), selected token ids and masks exactly."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import spa as OS
from _helpers import cpu

pytestmark = pytest.mark.gpu


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
        self.key = torch.full((n,), 9.0, **f64)
        self.proxy = torch.empty(n, r, **f64)
        self.mask = torch.full((n,), 7, device="cuda", dtype=torch.uint8)
        self.selected = torch.full((max(n_select, 1),), -1, device="cuda", dtype=torch.int32)
        self.d = d

    def step(self, x, f, init, with_proxy=True):
        fb = self.fb
        a = fb.proxy_args(x, f, self.cache, self.mask, self.selected, self.n_select, init,
                          key=self.key, proxy=self.proxy if with_proxy else None)
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
]


@pytest.mark.parametrize("name,n,d,r,k,dt", CASES, ids=[c[0] for c in CASES])
def test_identifier_matches_oracle_bit_for_bit(fb, name, n, d, r, k, dt):
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
    for s, (x, rec) in enumerate(zip(steps, recs)):
        idn.step(_dev(x, dt), f_d, init=(s == 0))
        tag = "%s step %d" % (name, s)
        assert np.array_equal(cpu(idn.proxy), rec["proxy"]), tag
        assert np.array_equal(cpu(idn.cache), rec["cache"]), tag
        assert np.array_equal(cpu(idn.mask).astype(bool), rec["mask"]), tag
        if s > 0:
            assert np.array_equal(cpu(idn.key), rec["key"]), tag
            if k > 0:
                assert np.array_equal(cpu(idn.selected)[:k], rec["selected"]), tag


def test_identifier_sums_in_blocks_of_128(fb):
    # 2^53 at c = 0, ones at c = 128 and 129, a factor of ones: the blocked
    # sum is 2^53 + 2 exactly; a single running sum would give 2^53
    d, r = 256, 32
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 2.0 ** 53
    x[0, 128] = x[0, 129] = 1.0
    f = np.ones((d, r), np.float32)
    idn = Ident(fb, 1, d, r, 0)
    idn.step(_dev(W.bf16_bits(x), "bf16"), _dev(W.bf16_bits(f), "bf16"), init=True)
    assert (cpu(idn.proxy) == 2.0 ** 53 + 2.0).all()
    assert (cpu(idn.proxy) == OS.proxy(x, f)).all()


def test_identifier_ties_go_to_lower_ids(fb):
    # every token identical and its cache identical: all keys are 1 exactly
    n, d, r, k = 50, 512, 32, 9
    rng = np.random.default_rng(0)
    row = W.bf16_bits(rng.standard_normal((1, d)).astype(np.float32))
    x = np.repeat(row, n, axis=0)
    f = W.spa_factor(W.SPA.with_(d_model=d, rank=r))
    idn = Ident(fb, n, d, r, k)
    idn.step(_dev(x, "bf16"), _dev(f, "bf16"), init=True)
    idn.step(_dev(x, "bf16"), _dev(f, "bf16"), init=False, with_proxy=False)
    assert (cpu(idn.key) == 1.0).all()
    assert cpu(idn.selected)[:k].tolist() == list(range(k))


def test_identifier_full_size_bit_exact(fb):
    """1024 tokens of width 4096, rank 128, a quarter recomputed per step --
    the size the benchmark times."""
    cfg = W.SPA.with_(n_steps=2)
    f = W.spa_factor(cfg)
    steps = W.spa_steps(cfg)
    recs = OS.spa_run([W.values(x, "bf16") for x in steps], W.values(f, "bf16"), cfg.n_select)
    idn = Ident(fb, cfg.n_tok, cfg.d_model, cfg.rank, cfg.n_select)
    f_d = _dev(f, "bf16")
    for s, (x, rec) in enumerate(zip(steps, recs)):
        idn.step(_dev(x, "bf16"), f_d, init=(s == 0))
        assert np.array_equal(cpu(idn.proxy), rec["proxy"]), s
        assert np.array_equal(cpu(idn.cache), rec["cache"]), s
    assert np.array_equal(cpu(idn.key), recs[1]["key"])
    assert np.array_equal(cpu(idn.selected), recs[1]["selected"])


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
        recs = OS.spa_run([W.values(x, "bf16") for x in steps], W.values(f, "bf16"), counts[layer])
        idn = Ident(fb, n, d, r, counts[layer])
        f_d = _dev(f, "bf16")
        for s, (x, rec) in enumerate(zip(steps, recs)):
            idn.step(_dev(x, "bf16"), f_d, init=(s == 0))
            assert np.array_equal(cpu(idn.cache), rec["cache"]), (layer, s)
            assert np.array_equal(cpu(idn.mask).astype(bool), rec["mask"]), (layer, s)
