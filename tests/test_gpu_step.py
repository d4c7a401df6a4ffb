"""GPU parity of whole FlashBlock blocks driven by fb_step (text, video,
sparse) against the oracle's per-step paths: decisions and counts bit for
bit, outputs to tolerance, every step."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from _helpers import check_a, check_l, cpu, dev_tensor, tols, vals

pytestmark = pytest.mark.gpu


def run_text(fb, cfg, m_override=None, layout="tok", force=None):
    steps = W.text_steps(cfg, m_override=m_override)
    kp, vp = W.prefix_kv(cfg)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, tdt)
    step = fb.Step(fb.FB_STEP_TEXT, shape, cfg.n_block, dev_tensor(kp, cfg.dtype, layout),
                   dev_tensor(vp, cfg.dtype, layout), tau=cfg.tau)
    got = []
    for s, st in enumerate(steps):
        a = torch.empty(cfg.n_block, cfg.n_q_heads, cfg.head_dim, device="cuda")
        l = torch.empty(cfg.n_block, cfg.n_q_heads, device="cuda")
        dec = -1
        if force is not None and s > 0 and force[s] is not None:
            dec = 1 if force[s] == OC.REUSE else 0
        step.step(dev_tensor(st["q"], cfg.dtype), dev_tensor(st["k"], cfg.dtype),
                  dev_tensor(st["v"], cfg.dtype), a, l,
                  ids=torch.from_numpy(st["ids"]).cuda(), decision=dec)
        got.append((cpu(a), cpu(l), int(step.m_count.item()), cpu(step.mask), cpu(step.a_out)))
    ksteps = [dict(q=vals(s["q"], cfg.dtype), k=vals(s["k"], cfg.dtype),
                   v=vals(s["v"], cfg.dtype), ids=s["ids"]) for s in steps]
    recs = OC.text_block(ksteps, vals(kp, cfg.dtype), vals(vp, cfg.dtype), cfg.scale, cfg.tau,
                         with_dense=False, force=force)
    return got, recs


@pytest.mark.parametrize("name,cfg,m_override", [
    ("tiny_f32", W.TINY, None),
    ("text_b4_32k", W.TEXT, None),
    ("text_b4_forced_M", W.TEXT.with_(n_prefix=9000, n_steps=8), [None, 0, 1, 2, 4, 1, 0, 3]),
    ("long_b16_small", W.LONG.with_(n_prefix=40000), None),
    ("long_b8_small", W.LONG.with_(n_prefix=40000, n_block=8), None),
])
def test_text_block_matches_oracle(fb, name, cfg, m_override):
    got, recs = run_text(fb, cfg, m_override)
    atol, ltol = tols(cfg.dtype)
    for s, (rec, (a, l, mc, mask, a_out)) in enumerate(zip(recs, got)):
        if s > 0:
            assert mc == rec["m_count"], (s, mc, rec["m_count"])
        assert np.all(mask == (1 if rec["decision"] == OC.REUSE else 0)), (s, rec["decision"])
        check_a("%s step %d A_out" % (name, s), a_out, rec["a_out"], atol)
        check_a("%s step %d A_full" % (name, s), a, rec["a_full"], atol)
        check_l("%s step %d L_full" % (name, s), l, rec["l_full"], ltol)


def test_text_forced_reuse_and_recompute(fb):
    cfg = W.TEXT.with_(n_prefix=5000, n_steps=5)
    force = [None, OC.REUSE, OC.RECOMPUTE, OC.REUSE, OC.REUSE]
    got, recs = run_text(fb, cfg, m_override=[None, 4, 0, 4, 4], force=force)
    for s, (rec, (a, l, mc, mask, a_out)) in enumerate(zip(recs, got)):
        assert rec["decision"] == ([OC.INIT] + force[1:])[s]
        check_a("forced step %d" % s, a, rec["a_full"], 2e-3)
        check_l("forced step %d" % s, l, rec["l_full"], 1e-3)


def test_text_head_major_prefix(fb):
    cfg = W.LONG.with_(n_prefix=12345, n_steps=4)
    got, recs = run_text(fb, cfg, layout="head")
    for s, (rec, (a, l, *_)) in enumerate(zip(recs, got)):
        check_a("headmajor step %d" % s, a, rec["a_full"], 2e-3)


def _video_sigmas(cfg, variant, gamma, margin=1e-3, tries=20):
    """Redraw the per-head noise scales until no head's similarity lies within
    `margin` of gamma in the oracle (so the GPU's fp32 outputs decide alike)."""
    kp, vp = W.prefix_kv(cfg)
    for v in range(variant, variant + tries):
        sig = W.video_sigmas(cfg, v)
        steps = W.video_steps(cfg, sig)
        ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16")) for s in steps]
        recs = OC.video_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, gamma)
        sims = np.concatenate([r["sim"][~np.isnan(r["sim"])] for r in recs[1:]])
        if np.all(np.abs(sims - gamma) >= margin):
            return sig, steps, kp, vp, recs
    raise RuntimeError("no margin-clean sigma draw")


@pytest.mark.parametrize("n_q,n_kv", [(120, 300), (256, 640)])
def test_video_block_matches_oracle(fb, n_q, n_kv):
    cfg = W.VIDEO.with_(n_block=n_q, n_prefix=n_kv, n_steps=4)
    sig, steps, kp, vp, recs = _video_sigmas(cfg, 0, cfg.gamma)
    shape = fb.shape_of(12, 12, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_VIDEO, shape, n_q, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                   gamma=cfg.gamma)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        used = cpu(step.mask).copy() if s > 0 else np.zeros(12, np.uint8)
        a = torch.empty(n_q, 12, 128, device="cuda")
        l = torch.empty(n_q, 12, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        if s > 0:
            assert np.array_equal(used.astype(bool), rec["reuse_used"]), (s, used, rec["reuse_used"])
            assert np.array_equal(cpu(step.mask).astype(bool), rec["reuse_next"])
            ok = ~np.isnan(rec["sim"])
            assert np.allclose(cpu(step.sim)[ok], rec["sim"][ok], atol=1e-4)
        check_a("video step %d A_out" % s, cpu(step.a_out), rec["a_out"], 2e-3)
        check_a("video step %d A_full" % s, cpu(a), rec["a_full"], 2e-3)
        check_l("video step %d L_full" % s, cpu(l), rec["l_full"], 1e-3)


@pytest.mark.parametrize("density", [0.2, 0.4])
def test_sparse_block_matches_oracle(fb, density):
    cfg = W.SPARSE.with_(n_prefix=4096, density=density, n_steps=5)
    steps = W.sparse_steps(cfg, m_override=[None, 2, 0, 5, 1])
    kp, vp = W.prefix_kv(cfg)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_SPARSE, shape, 8, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                   page_size=cfg.page, k_pages=cfg.k_pages, pct=cfg.pct)
    ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16"))
          for s in steps]
    recs = OC.sparse_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, cfg.k_pages, cfg.page)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        a = torch.empty(8, 32, 128, device="cuda")
        l = torch.empty(8, 32, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        assert np.array_equal(cpu(step.pages), rec["sel"]), s
        assert np.array_equal(cpu(step.active).astype(bool), rec["active"]), s
        if s == 0:
            check_a("sparse A_res", cpu(step.a_res), rec["a_res"], 2e-3)
            check_l("sparse L_res", cpu(step.l_res), rec["l_res"], 1e-3)
        check_a("sparse step %d A_out" % s, cpu(step.a_out), rec["a_out"], 2e-3)
        check_a("sparse step %d A_full" % s, cpu(a), rec["a_full"], 2e-3)
        check_l("sparse step %d L_full" % s, cpu(l), rec["l_full"], 1e-3)
