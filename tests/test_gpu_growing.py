"""GPU parity of the outer loop over blocks: the finished block's K/V joins
the prefix cache (fb_kv_append, bit for bit), page metadata follows the
grown cache incrementally (fb_page_meta_update, bit for bit against the
oracle's metadata of the whole grown prefix), whole runs of several blocks
through fb_step / fb_step_next_block against oracle.growing.run_blocks
(decisions and counts bit for bit, outputs to tolerance), and the
count-since-refresh reading of M (fb_reuse_decide and fb_step)."""

import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from oracle import growing as OG
from oracle import quest as OQ
from _helpers import check_a, check_l, check_mse, cpu, dev_tensor, mse_margin_ok, tols, vals

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _torch_dt(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def _bits(t):
    """Raw element bits of a device tensor (bf16 -> int16, f32 -> int32)."""
    t = t.detach().cpu().contiguous()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).numpy()


def _strided(x, dtype):
    """Device copy of a [B, H, d] block whose token stride is padded (a
    non-contiguous source for the append)."""
    t = dev_tensor(x, dtype)
    b, h, d = t.shape
    big = torch.zeros(b, h + 1, d, device="cuda", dtype=t.dtype)
    big[:, :h] = t
    return big[:, :h]


@pytest.mark.parametrize("layout", ["head", "token"])
@pytest.mark.parametrize("cfg", [W.LONG.with_(n_kv_heads=8, head_dim=128),
                                 W.TINY.with_(n_kv_heads=4, head_dim=64)],
                         ids=["bf16_d128", "f32_d64"])
def test_kv_append_bit_exact(fb, cfg, layout):
    sizes = [37, 16, 5, 1, 16]                  # the first append fills the initial prefix
    cap = sum(sizes) + 3
    k_all, v_all = W.prefix_kv(cfg, n_tok=sum(sizes), variant=4)
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, _torch_dt(cfg))
    cache = fb.KVCache(cap, cfg.n_kv_heads, cfg.head_dim, _torch_dt(cfg), "cuda", layout)
    lo = 0
    for i, b in enumerate(sizes):
        kb, vb = k_all[lo:lo + b], v_all[lo:lo + b]
        if i % 2:
            cache.append(shape, _strided(kb, cfg.dtype), _strided(vb, cfg.dtype))
        else:
            cache.append(shape, dev_tensor(kb, cfg.dtype), dev_tensor(vb, cfg.dtype))
        lo += b
        assert cache.n_tok == lo
        torch.cuda.synchronize()
        assert np.array_equal(_bits(cache.k_prefix), _bits(dev_tensor(k_all[:lo], cfg.dtype)))
        assert np.array_equal(_bits(cache.v_prefix), _bits(dev_tensor(v_all[:lo], cfg.dtype)))
    # beyond the capacity: rejected, count unchanged, storage untouched
    blk = dev_tensor(k_all[:4], cfg.dtype)
    with pytest.raises(fb.FlashBlockError):
        cache.append(shape, blk, blk)
    assert cache.n_tok == lo


def test_kv_append_in_place_block(fb):
    """A block written straight into the cache's tail is taken as is."""
    cfg = W.LONG
    k_all, v_all = W.prefix_kv(cfg, n_tok=70, variant=6)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(80, 8, 128, torch.bfloat16, "cuda", "head")
    cache.append(shape, dev_tensor(k_all[:60], "bf16"), dev_tensor(v_all[:60], "bf16"))
    tail_k, tail_v = cache.k_all[60:70], cache.v_all[60:70]
    tail_k.copy_(dev_tensor(k_all[60:70], "bf16"))
    tail_v.copy_(dev_tensor(v_all[60:70], "bf16"))
    cache.append(shape, tail_k, tail_v)
    torch.cuda.synchronize()
    assert cache.n_tok == 70
    assert np.array_equal(_bits(cache.k_prefix), _bits(dev_tensor(k_all, "bf16")))
    assert np.array_equal(_bits(cache.v_prefix), _bits(dev_tensor(v_all, "bf16")))


@pytest.mark.parametrize("page", [16, 7])
def test_page_meta_update_bit_exact(fb, page):
    cfg = W.SPARSE
    grow = [0, 37, 38, 48, 64, 65, 200, 401]
    k_all, v_all = W.prefix_kv(cfg, n_tok=grow[-1], variant=2)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(grow[-1], 8, 128, torch.bfloat16, "cuda", "token")
    cap = (grow[-1] + page - 1) // page
    sentinel = -12288.0                 # exact in bf16
    kmin = torch.full((8, cap, 128), sentinel, device="cuda", dtype=torch.bfloat16)
    kmax = torch.full((8, cap, 128), sentinel, device="cuda", dtype=torch.bfloat16)
    for n_old, n_new in zip(grow[:-1], grow[1:]):
        cache.append(shape, dev_tensor(k_all[n_old:n_new], "bf16"),
                     dev_tensor(v_all[n_old:n_new], "bf16"))
        fb.fb_page_meta_update(shape, cache.k_prefix, page, n_old, cap, kmin, kmax)
        torch.cuda.synchronize()
        p = (n_new + page - 1) // page
        rmin, rmax = OQ.page_meta(vals(k_all[:n_new], "bf16"), page)
        gmin = kmin.float().cpu().numpy()
        gmax = kmax.float().cpu().numpy()
        assert np.array_equal(gmin[:, :p], rmin) and np.array_equal(gmax[:, :p], rmax), n_new
        assert (gmin[:, p:] == sentinel).all() and (gmax[:, p:] == sentinel).all(), n_new


def _step_inputs(cfg, steps):
    return [dict(q=vals(s["q"], cfg.dtype), k=vals(s["k"], cfg.dtype), v=vals(s["v"], cfg.dtype),
                 ids=s["ids"]) for s in steps]


@pytest.mark.parametrize("layout,since_refresh", [("head", False), ("token", False),
                                                  ("head", True)])
def test_text_blocks_on_a_growing_cache(fb, layout, since_refresh):
    cfg = W.LONG.with_(n_prefix=3001, n_block=16, n_steps=5, tau=3)
    n_blocks = 4
    kp, vp = W.prefix_kv(cfg, variant=1)
    blocks = [W.text_steps(cfg, variant=1, block=j) for j in range(n_blocks)]
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(cfg.n_prefix + n_blocks * 16, 8, 128, torch.bfloat16, "cuda", layout)
    cache.append(shape, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"))
    step = fb.Step(fb.FB_STEP_TEXT, shape, 16, cache=cache, tau=cfg.tau,
                   since_refresh=since_refresh)
    out, (kc, vc) = OG.run_blocks([_step_inputs(cfg, b) for b in blocks], vals(kp, "bf16"),
                                  vals(vp, "bf16"), OC.text_block, scale=cfg.scale, tau=cfg.tau,
                                  with_dense=False, since_refresh=since_refresh)
    n_recompute = 0
    for j, (steps, blk) in enumerate(zip(blocks, out)):
        assert step.state.k_prefix.n_tok == blk["n_prefix"]
        for s, (st, rec) in enumerate(zip(steps, blk["recs"])):
            a = torch.empty(16, 32, 128, device="cuda")
            l = torch.empty(16, 32, device="cuda")
            step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                      dev_tensor(st["v"], "bf16"), a, l, ids=torch.from_numpy(st["ids"]).cuda())
            torch.cuda.synchronize()
            tag = "block %d step %d" % (j, s)
            if s > 0:
                assert int(step.m_count.item()) == rec["m_count"], tag
                n_recompute += rec["decision"] == OC.RECOMPUTE
            assert np.all(cpu(step.mask) == (1 if rec["decision"] == OC.REUSE else 0)), tag
            check_a(tag + " A_out", cpu(step.a_out), rec["a_out"], 2e-3)
            check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
            check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)
        step.next_block(dev_tensor(steps[-1]["k"], "bf16"), dev_tensor(steps[-1]["v"], "bf16"))
        assert step.state.step == 0
    assert n_recompute > 0
    torch.cuda.synchronize()
    assert cache.n_tok == kc.shape[0]
    assert np.array_equal(cache.k_prefix.float().cpu().numpy(), kc)
    assert np.array_equal(cache.v_prefix.float().cpu().numpy(), vc)


def test_sparse_blocks_on_a_growing_cache(fb):
    cfg = W.SPARSE.with_(n_prefix=4001, n_block=8, n_steps=3)
    n_blocks, k_pages = 3, 60
    kp, vp = W.prefix_kv(cfg, variant=2)
    blocks = [W.sparse_steps(cfg, variant=2, block=j, m_override=[None, 3, 1])
              for j in range(n_blocks)]
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(cfg.n_prefix + n_blocks * 8, 8, 128, torch.bfloat16, "cuda", "head")
    cache.append(shape, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"))
    step = fb.Step(fb.FB_STEP_SPARSE, shape, 8, cache=cache, page_size=16, k_pages=k_pages,
                   pct=cfg.pct)
    inputs = [[dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16"))
               for s in b] for b in blocks]
    out, _ = OG.run_blocks(inputs, vals(kp, "bf16"), vals(vp, "bf16"), OC.sparse_block,
                           scale=cfg.scale, k_pages=k_pages, page=16)
    for j, (steps, blk) in enumerate(zip(blocks, out)):
        n_j = blk["n_prefix"]
        for s, (st, rec) in enumerate(zip(steps, blk["recs"])):
            a = torch.empty(8, 32, 128, device="cuda")
            l = torch.empty(8, 32, device="cuda")
            step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                      dev_tensor(st["v"], "bf16"), a, l)
            torch.cuda.synchronize()
            tag = "block %d step %d" % (j, s)
            assert np.array_equal(cpu(step.pages), rec["sel"]), tag
            if s > 0:
                assert mse_margin_ok(rec["mse"]), tag
                check_mse(tag, cpu(step.mse), rec["mse"])
            assert np.array_equal(cpu(step.active).astype(bool), rec["active"]), tag
            check_a(tag + " A_out", cpu(step.a_out), rec["a_out"], 2e-3)
            check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
            check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)
        # the metadata the next refresh selects from is the grown prefix's
        step.next_block(dev_tensor(steps[-1]["k"], "bf16"), dev_tensor(steps[-1]["v"], "bf16"))
        torch.cuda.synchronize()
        n_next = n_j + 8
        p = (n_next + 15) // 16
        kc = np.concatenate([vals(kp, "bf16")] +
                            [vals(blocks[i][-1]["k"], "bf16") for i in range(j + 1)])
        rmin, rmax = OQ.page_meta(kc, 16)
        assert np.array_equal(step.kmin.float().cpu().numpy()[:, :p], rmin), j
        assert np.array_equal(step.kmax.float().cpu().numpy()[:, :p], rmax), j


def test_count_since_refresh_hand_fixture(fb):
    g = json.load(open(os.path.join(GOLD, "text_controller_since_refresh.json")))
    ids = [torch.tensor(x, dtype=torch.int32, device="cuda") for x in g["ids"]]
    n = len(g["ids"][0])
    for mode in ("per_step", "since_refresh"):
        kept = ids[0].clone()
        mask = torch.zeros(8, dtype=torch.uint8, device="cuda")
        m = torch.zeros(1, dtype=torch.int32, device="cuda")
        for s in range(1, len(ids)):
            a = fb.fb_reuse_args()
            a.mode, a.n_q, a.n_heads = fb.FB_REUSE_COUNT, n, 8
            a.ids_prev, a.ids_cur, a.tau, a.force = kept.data_ptr(), ids[s].data_ptr(), g["tau"], -1
            a.m_count, a.ids_store, a.mask = m.data_ptr(), kept.data_ptr(), mask.data_ptr()
            a.since_refresh = 1 if mode == "since_refresh" else 0
            fb.fb_reuse_decide(a)
            torch.cuda.synchronize()
            assert int(m.item()) == g[mode]["m_count"][s], (mode, s)
            want = 1 if g[mode]["decision"][s] == "reuse" else 0
            assert (cpu(mask) == want).all(), (mode, s)


def test_since_refresh_with_forced_decisions(fb):
    """Forced reuse keeps the ids of the last recompute; forced recompute
    takes the step's ids: M counted since the refresh follows both."""
    cfg = W.LONG.with_(n_prefix=2000, n_block=16, n_steps=6, tau=3)
    steps = W.text_steps(cfg, variant=2, m_override=[None, 2, 1, 1, 4, 1])
    kp, vp = W.prefix_kv(cfg, variant=2)
    force = [None, OC.REUSE, OC.RECOMPUTE, OC.REUSE, None, None]
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_TEXT, shape, 16, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                   tau=cfg.tau, since_refresh=True)
    recs = OC.text_block(_step_inputs(cfg, steps), vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale,
                         cfg.tau, with_dense=False, force=force, since_refresh=True)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        a = torch.empty(16, 32, 128, device="cuda")
        l = torch.empty(16, 32, device="cuda")
        dec = -1 if force[s] is None else (1 if force[s] == OC.REUSE else 0)
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l, ids=torch.from_numpy(st["ids"]).cuda(),
                  decision=dec)
        torch.cuda.synchronize()
        if s > 0:
            assert int(step.m_count.item()) == rec["m_count"], s
        assert np.all(cpu(step.mask) == (1 if rec["decision"] == OC.REUSE else 0)), s
        check_a("forced since-refresh step %d" % s, cpu(a), rec["a_full"], 2e-3)


def test_append_fills_the_cache_exactly(fb):
    cfg = W.LONG
    k_all, v_all = W.prefix_kv(cfg, n_tok=48, variant=5)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    for layout in ("head", "token"):
        cache = fb.KVCache(48, 8, 128, torch.bfloat16, "cuda", layout)
        cache.append(shape, dev_tensor(k_all[:32], "bf16"), dev_tensor(v_all[:32], "bf16"))
        # a head-major block as the source
        cache.append(shape, dev_tensor(k_all[32:], "bf16", "head"),
                     dev_tensor(v_all[32:], "bf16", "head"))
        torch.cuda.synchronize()
        assert cache.n_tok == 48
        assert np.array_equal(_bits(cache.k_prefix), _bits(dev_tensor(k_all, "bf16")))
        assert np.array_equal(_bits(cache.v_prefix), _bits(dev_tensor(v_all, "bf16")))
        blk = dev_tensor(k_all[:1], "bf16")
        with pytest.raises(fb.FlashBlockError):
            cache.append(shape, blk, blk)


def test_video_blocks_on_a_growing_cache(fb):
    """Video mode (12 MHA heads, 256 block queries: the many-rows MFMA pass)
    over a head-major cache of fixed capacity that takes each finished block:
    per-head decisions and outputs against the oracle's growing run. The
    per-head noise scales are redrawn until no head's similarity lies within
    1e-3 of gamma, so both sides decide alike."""
    cfg = W.VIDEO.with_(n_prefix=1500, n_block=256, n_steps=3)
    n_blocks = 2
    for variant in range(3, 20):
        sig = W.video_sigmas(cfg, variant)
        kp, vp = W.prefix_kv(cfg, variant=variant)
        blocks = [W.video_steps(cfg, sig, variant=variant, block=j) for j in range(n_blocks)]
        inputs = [[dict(q=vals(x["q"], "bf16"), k=vals(x["k"], "bf16"), v=vals(x["v"], "bf16"))
                   for x in b] for b in blocks]
        out, _ = OG.run_blocks(inputs, vals(kp, "bf16"), vals(vp, "bf16"), OC.video_block,
                               scale=cfg.scale, gamma=cfg.gamma)
        sims = np.concatenate([r["sim"] for b in out for r in b["recs"]])
        sims = sims[~np.isnan(sims)]
        if (np.abs(sims - cfg.gamma) > 1e-3).all():
            break
    shape = fb.shape_of(12, 12, 128, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(cfg.n_prefix + n_blocks * 256, 12, 128, torch.bfloat16, "cuda", "head")
    cache.append(shape, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"))
    step = fb.Step(fb.FB_STEP_VIDEO, shape, 256, cache=cache, gamma=cfg.gamma)
    n_reused = 0
    for j, (steps, blk) in enumerate(zip(blocks, out)):
        for s, (st, rec) in enumerate(zip(steps, blk["recs"])):
            # the state holds the flags the coming step uses; after a step,
            # those of the next one
            used = cpu(step.mask).astype(bool) if s > 0 else np.zeros(12, bool)
            a = torch.empty(256, 12, 128, device="cuda")
            l = torch.empty(256, 12, device="cuda")
            step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                      dev_tensor(st["v"], "bf16"), a, l)
            torch.cuda.synchronize()
            tag = "block %d step %d" % (j, s)
            assert np.array_equal(used, rec["reuse_used"]), tag
            if s > 0:
                assert np.array_equal(cpu(step.mask).astype(bool), rec["reuse_next"]), tag
            n_reused += int(used.sum())
            check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
            check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)
        step.next_block(dev_tensor(steps[-1]["k"], "bf16"), dev_tensor(steps[-1]["v"], "bf16"))
    assert cache.n_tok == cfg.n_prefix + n_blocks * 256
    assert n_reused > 0
