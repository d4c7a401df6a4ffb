"""GPU parity at the sizes and launch configurations the benchmark times,
element by element against the oracle (head-major prefix K/V, as timed):

* the 800,000-token prefix pass (B = 16, 32q/8kv, d = 128): all 512 rows,
  on head-major and on token-major K/V;
* the 800,000-token text block through fb_step (8 steps, tau = 4): every
  row of two whole KV groups, every step: count, decision, the cached pair
  and the merged output;
* the video block through fb_step (4,680 block queries, 12,480 prefix
  tokens, 12 heads, 4 steps, gamma = 0.95): per-head flags every step (the
  noise scales are those the benchmark draws, checked to leave every
  similarity at least 1e-3 from gamma), every output element of every head;
* the sparse FlashBlock block (65,536-token prefix, 16-token pages, B = 8,
  8 steps) at densities 0.2, 0.3 and 0.4, and LoSA's own step at the same
  densities: pages and active sets bit for bit (the query MSEs leave a
  margin, asserted per step), every output element.

The oracle computes one KV group at a time in float64 over every key.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from oracle.attention import attn
from _helpers import check_a, check_l, check_mse, cpu, dev_tensor, mse_margin_ok, vals

pytestmark = pytest.mark.gpu

N_TEXT, B_TEXT = 800000, 16


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def text_800k():
    cfg = W.LONG.with_(n_prefix=N_TEXT, n_block=B_TEXT)
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    return cfg, kp, vp, steps


def test_text_800k_prefix_pass_all_rows(fb, text_800k):
    cfg, kp, vp, steps = text_800k
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = hq // hkv
    q = steps[0]["q"]
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, B_TEXT, N_TEXT), 16),
                     dtype=torch.uint8, device="cuda")
    got = {}
    for layout in ("head", "token"):
        _say("800k prefix pass, %s-major K/V" % layout)
        kd, vd = dev_tensor(kp, "bf16", layout), dev_tensor(vp, "bf16", layout)
        a = torch.empty(B_TEXT, hq, d, device="cuda")
        l = torch.empty(B_TEXT, hq, device="cuda")
        fb.fb_prefix_attn(shape, dev_tensor(q, "bf16"), kd, vd, a, l, ws=ws)
        torch.cuda.synchronize()
        got[layout] = (cpu(a), cpu(l))
        del kd, vd
        torch.cuda.empty_cache()
    for g in range(hkv):
        heads = list(range(g * G, (g + 1) * G))
        qr = vals(q[:, heads, :], "bf16").reshape(-1, d)          # rows (t, h) of the group
        ra, rl = attn(qr, vals(kp[:, g, :], "bf16"), vals(vp[:, g, :], "bf16"), cfg.scale)
        ra, rl = ra.reshape(B_TEXT, G, d), rl.reshape(B_TEXT, G)
        for layout, (a, l) in got.items():
            check_a("800k %s group %d A_out" % (layout, g), a[:, heads], ra, 2e-3)
            check_l("800k %s group %d L_out" % (layout, g), l[:, heads], rl, 1e-3)


def test_text_800k_block_two_groups_every_row(fb, text_800k):
    cfg, kp, vp, steps = text_800k
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = hq // hkv
    groups = (0, 5)
    heads = [h for g in groups for h in range(g * G, (g + 1) * G)]
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_TEXT, shape, B_TEXT, dev_tensor(kp, "bf16", "head"),
                   dev_tensor(vp, "bf16", "head"), tau=cfg.tau)
    got = []
    for s, st in enumerate(steps):
        a = torch.empty(B_TEXT, hq, d, device="cuda")
        l = torch.empty(B_TEXT, hq, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l, ids=torch.from_numpy(st["ids"]).cuda())
        torch.cuda.synchronize()
        got.append((cpu(a)[:, heads], cpu(l)[:, heads], int(step.m_count.item()), cpu(step.mask),
                    cpu(step.a_out)[:, heads], cpu(step.l_out)[:, heads]))
    # the oracle on the two groups alone: query heads `heads`, KV heads `groups`
    # (the sub-model keeps the contiguous 4:1 head mapping)
    _say("800k block: oracle over KV groups %s" % (groups,))
    sub = [dict(q=vals(st["q"][:, heads], "bf16"), k=vals(st["k"][:, list(groups)], "bf16"),
                v=vals(st["v"][:, list(groups)], "bf16"), ids=st["ids"]) for st in steps]
    recs = OC.text_block(sub, vals(kp[:, list(groups)], "bf16"), vals(vp[:, list(groups)], "bf16"),
                         cfg.scale, cfg.tau, with_dense=False)
    for s, (rec, (a, l, mc, mask, a_out, l_out)) in enumerate(zip(recs, got)):
        tag = "800k block step %d" % s
        if s > 0:
            assert mc == rec["m_count"], (tag, mc, rec["m_count"])
        assert np.all(mask == (1 if rec["decision"] == OC.REUSE else 0)), (tag, rec["decision"])
        check_a(tag + " A_out", a_out, rec["a_out"], 2e-3)
        check_l(tag + " L_out", l_out, rec["l_out"], 1e-3)
        check_a(tag + " A_full", a, rec["a_full"], 2e-3)
        check_l(tag + " L_full", l, rec["l_full"], 1e-3)
    assert {r["decision"] for r in recs[1:]} == {OC.REUSE, OC.RECOMPUTE}


def test_video_block_full_size(fb):
    cfg = W.VIDEO
    H, d, NQ = cfg.n_q_heads, cfg.head_dim, cfg.n_block
    kp, vp = W.prefix_kv(cfg)
    sig = W.video_sigmas(cfg, 0)                   # the noise scales the benchmark draws
    steps = W.video_steps(cfg, sig)
    _say("video block: oracle, 4 steps")
    ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16")) for s in steps]
    recs = OC.video_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, cfg.gamma)
    sims = np.concatenate([r["sim"][~np.isnan(r["sim"])] for r in recs[1:]])
    assert np.all(np.abs(sims - cfg.gamma) >= 1e-3), "a similarity lies within 1e-3 of gamma"
    shape = fb.shape_of(H, H, d, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_VIDEO, shape, NQ, dev_tensor(kp, "bf16", "head"),
                   dev_tensor(vp, "bf16", "head"), gamma=cfg.gamma)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        _say("video block: GPU step %d" % s)
        used = cpu(step.mask).copy() if s > 0 else np.zeros(H, np.uint8)
        a = torch.empty(NQ, H, d, device="cuda")
        l = torch.empty(NQ, H, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        tag = "video step %d" % s
        if s > 0:
            assert np.array_equal(used.astype(bool), rec["reuse_used"]), (tag, used, rec["reuse_used"])
            assert np.array_equal(cpu(step.mask).astype(bool), rec["reuse_next"]), tag
            ok = ~np.isnan(rec["sim"])
            assert np.max(np.abs(cpu(step.sim)[ok] - rec["sim"][ok])) < 1e-4, tag
        check_a(tag + " A_out", cpu(step.a_out), rec["a_out"], 2e-3)
        check_l(tag + " L_out", cpu(step.l_out), rec["l_out"], 1e-3)
        check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
        check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)
    assert any(r["reuse_used"].any() for r in recs[2:]) and not all(r["reuse_used"].all() for r in recs[2:])


@pytest.fixture(scope="module")
def sparse_64k():
    cfg = W.SPARSE
    kp, vp = W.prefix_kv(cfg)
    return cfg, kp, vp, vals(kp, "bf16"), vals(vp, "bf16")


def _sparse_run(fb, cfg, kp, vp, steps, reselect):
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_SPARSE, shape, 8, dev_tensor(kp, "bf16", "head"),
                   dev_tensor(vp, "bf16", "head"), page_size=cfg.page, k_pages=cfg.k_pages,
                   pct=cfg.pct, reselect=reselect)
    out = []
    for st in steps:
        a = torch.empty(8, 32, 128, device="cuda")
        l = torch.empty(8, 32, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        out.append(dict(a=cpu(a), l=cpu(l), pages=cpu(step.pages), active=cpu(step.active).astype(bool),
                        mse=cpu(step.mse), a_out=cpu(step.a_out), l_out=cpu(step.l_out),
                        a_res=cpu(step.a_res), l_res=cpu(step.l_res)))
    return out


def _check_sparse_step(tag, g, rec, s, losa):
    if s > 0:
        assert mse_margin_ok(rec["mse"]), tag + ": query MSEs within the margin"
        check_mse(tag, g["mse"], rec["mse"])
    act = rec["active"]
    assert np.array_equal(g["active"], act), (tag, g["active"], act)
    if losa and s > 0:                             # pages are chosen for active tokens only
        assert np.array_equal(g["pages"][act], rec["sel"][act]), tag
    elif not losa:
        assert np.array_equal(g["pages"], rec["sel"]), tag
    if not losa and s == 0:
        check_a(tag + " A_res", g["a_res"], rec["a_res"], 2e-3)
        check_l(tag + " L_res", g["l_res"], rec["l_res"], 1e-3)
    check_a(tag + " A_out", g["a_out"], rec["a_out"], 2e-3)
    check_l(tag + " L_out", g["l_out"], rec["l_out"], 1e-3)
    check_a(tag + " A_full", g["a"], rec["a_full"], 2e-3)
    check_l(tag + " L_full", g["l"], rec["l_full"], 1e-3)


@pytest.mark.parametrize("density", W.SPARSE_DENSITIES)
@pytest.mark.parametrize("losa", [False, True], ids=["flashblock", "losa"])
def test_sparse_block_64k(fb, sparse_64k, density, losa):
    base, kp, vp, kv, vv = sparse_64k
    cfg = base.with_(density=density)
    steps = W.sparse_steps(cfg)                    # the block the benchmark times
    _say("sparse 64k density %.1f %s: GPU" % (density, "losa" if losa else "flashblock"))
    got = _sparse_run(fb, cfg, kp, vp, steps, losa)
    _say("sparse 64k: oracle")
    ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16")) for s in steps]
    block = OC.losa_block if losa else OC.sparse_block
    recs = block(ks, kv, vv, cfg.scale, cfg.k_pages, cfg.page, cfg.pct)
    for s, (g, rec) in enumerate(zip(got, recs)):
        _check_sparse_step("sparse 64k d%.1f %s step %d" % (density, "losa" if losa else "fb", s),
                           g, rec, s, losa)
    assert any(0 < r["active"].sum() < 8 for r in recs[1:])
