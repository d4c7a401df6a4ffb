"""GPU parity of LoSA's per-step variant: the GATHER pass with no residual
(the pair over each active row's selected pages alone) against the oracle's
split attention, whole blocks through fb_step with sparse_reselect (pages
chosen with each step's queries: bit for bit; active sets bit for bit;
outputs to tolerance) against oracle.controller.losa_block, and selection
per query head through fb_page_select on per-head metadata against the
oracle's per-head bound and top-k."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from oracle import quest as OQ
from _helpers import check_a, check_l, check_mse, cpu, dev_tensor, mse_margin_ok, vals

pytestmark = pytest.mark.gpu


def _selection(rng, n_q, hkv, n_pages, k):
    return np.stack([np.stack([np.sort(rng.choice(n_pages, size=k, replace=False))
                               for _ in range(hkv)]) for _ in range(n_q)]).astype(np.int32)


GATHER_CASES = [
    # name, dtype, d, n_q, n_kv, page, k, active
    ("mfma_b8_ragged", "bf16", 128, 8, 20007, 16, 250, [1, 0, 1, 1, 0, 0, 1, 0]),
    ("mfma_b8_all_active", "bf16", 128, 8, 4096, 16, 64, [1] * 8),
    ("mfma_b8_none_active", "bf16", 128, 8, 4096, 16, 64, [0] * 8),
    ("mfma_k0", "bf16", 128, 4, 3000, 16, 0, [1, 1, 0, 1]),
    ("generic_page8", "bf16", 128, 8, 5001, 8, 100, [0, 1, 1, 0, 1, 0, 0, 1]),
    ("generic_f32_d64", "f32", 64, 4, 3000, 16, 30, [1, 0, 1, 1]),
]


@pytest.mark.parametrize("name,dt,d,n_q,n_kv,page,k,active", GATHER_CASES,
                         ids=[c[0] for c in GATHER_CASES])
def test_gather_without_residual(fb, name, dt, d, n_q, n_kv, page, k, active):
    cfg = W.SPARSE.with_(n_prefix=n_kv, n_block=n_q, n_steps=1, head_dim=d, dtype=dt,
                         cfg_id=5 if dt == "bf16" else 1)
    kp, vp = W.prefix_kv(cfg)
    q = W.text_steps(cfg)[0]["q"]
    n_pages = -(-n_kv // page)
    sel = _selection(np.random.default_rng(3), n_q, 8, n_pages, k)
    act = np.array(active, dtype=bool)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    shape = fb.shape_of(32, 8, d, cfg.scale, tdt)
    # page_sel keeps raw pointers: the tensors must outlive the call
    pages_d = torch.from_numpy(sel).cuda() if k > 0 else None
    act_d = torch.from_numpy(act.astype(np.uint8)).cuda()
    s = fb.page_sel(fb.FB_SEL_GATHER, page, pages_d, act_d)
    a = torch.full((n_q, 32, d), 7.0, device="cuda")
    l = torch.full((n_q, 32), 7.0, device="cuda")
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, n_q, n_kv, s), 16), dtype=torch.uint8,
                     device="cuda")
    fb.fb_prefix_attn(shape, dev_tensor(q, dt), dev_tensor(kp, dt), dev_tensor(vp, dt), a, l,
                      sel=s, ws=ws)
    torch.cuda.synchronize()
    a, l = cpu(a), cpu(l)
    assert (a[~act] == 7.0).all() and (l[~act] == 7.0).all()
    rows = np.nonzero(act)[0]
    if rows.size == 0:
        return
    (ra, rl), _ = OQ.split_attn(vals(q[rows], dt), vals(kp, dt), vals(vp, dt), sel[rows], page,
                                cfg.scale, residual=False)
    atol = 2e-3 if dt == "bf16" else 1e-5
    check_a(name + " A_sel", a[rows], ra, atol)
    check_l(name + " L_sel", l[rows], rl, 1e-3 if dt == "bf16" else 1e-5)


LOSA_CASES = [
    ("d02_4096", 4096, 0.2, [None, 2, 0, 5, 1]),
    ("d04_ragged", 4001, 0.4, [None, 3, 1, 8, 0]),
]


@pytest.mark.parametrize("sel_bitmap", [True, False], ids=["topk_bitmaps", "prep_each_step"])
@pytest.mark.parametrize("name,n_prefix,density,m_override", LOSA_CASES,
                         ids=[c[0] for c in LOSA_CASES])
def test_losa_block_matches_oracle(fb, name, n_prefix, density, m_override, sel_bitmap):
    # sel_bitmap: each step's top-k writes its selection as bitmaps and the
    # GATHER workgroups take the union (True), or a selection prep builds
    # them (False)
    cfg = W.SPARSE.with_(n_prefix=n_prefix, density=density, n_steps=len(m_override))
    steps = W.sparse_steps(cfg, variant=7, m_override=m_override)
    kp, vp = W.prefix_kv(cfg, variant=7)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_SPARSE, shape, 8, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                   page_size=cfg.page, k_pages=cfg.k_pages, pct=cfg.pct, reselect=True,
                   sel_bitmap=sel_bitmap)
    ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16"))
          for s in steps]
    recs = OC.losa_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, cfg.k_pages,
                         cfg.page, cfg.pct)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        a = torch.empty(8, 32, 128, device="cuda")
        l = torch.empty(8, 32, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        tag = "%s step %d" % (name, s)
        act = rec["active"]
        if s > 0:
            assert mse_margin_ok(rec["mse"]), tag
            check_mse(tag, cpu(step.mse), rec["mse"])
        assert np.array_equal(cpu(step.active).astype(bool), act), tag
        if s > 0:                                # pages are chosen for active tokens only
            assert np.array_equal(cpu(step.pages)[act], rec["sel"][act]), tag
        if s > 0 and sel_bitmap:                 # the top-k's bitmaps of the same pages
            bm = cpu(step.sel_bitmap).view(np.uint32)
            want = np.zeros_like(bm)
            for t in np.nonzero(act)[0]:
                for g in range(8):
                    for pg in rec["sel"][t][g]:
                        want[t, g, pg // 32] |= np.uint32(1) << np.uint32(pg % 32)
            assert np.array_equal(bm[act], want[act]), tag
        check_a(tag + " A_out", cpu(step.a_out), rec["a_out"], 2e-3)
        check_l(tag + " L_out", cpu(step.l_out), rec["l_out"], 1e-3)
        check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
        check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)


def test_selection_per_query_head_bit_exact(fb):
    """Selection with one page set per query head: the per-head bound is the
    group bound of a model whose every query head has its own KV head, so
    fb_page_select on metadata repeated per query head computes it."""
    cfg = W.SPARSE.with_(n_prefix=3001, n_steps=2)
    kp, _ = W.prefix_kv(cfg, variant=8)
    q = W.sparse_steps(cfg, variant=8)[1]["q"]
    page, k = 16, 40
    n_pages = -(-3001 // page)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    kmin = torch.empty(8, n_pages, 128, device="cuda", dtype=torch.bfloat16)
    kmax = torch.empty_like(kmin)
    fb.fb_page_meta(shape, dev_tensor(kp, "bf16"), page, kmin, kmax)
    per_head = fb.shape_of(32, 32, 128, cfg.scale, torch.bfloat16)
    kmin_h = kmin.repeat_interleave(4, dim=0).contiguous()
    kmax_h = kmax.repeat_interleave(4, dim=0).contiguous()
    pages = torch.empty(8, 32, k, device="cuda", dtype=torch.int32)
    ws = torch.empty(max(fb.fb_page_select_workspace(per_head, 8, n_pages), 16),
                     dtype=torch.uint8, device="cuda")
    fb.fb_page_select(per_head, dev_tensor(q, "bf16"), kmin_h, kmax_h, n_pages, k, pages, ws=ws)
    torch.cuda.synchronize()
    rmin, rmax = OQ.page_meta(vals(kp, "bf16"), page)
    ref = OQ.topk_pages(OQ.page_bound_heads(vals(q, "bf16"), rmin, rmax), k)
    got = cpu(pages)
    assert np.array_equal(got, ref)
    act = np.array([1, 0, 1, 1, 0, 1, 0, 0], dtype=bool)
    assert np.array_equal(OQ.union_size_heads(got, act, 8), OQ.union_size_heads(ref, act, 8))


def test_selection_of_active_tokens_only(fb):
    """fb_page_select with an active mask scores and selects the active
    tokens' rows (bit for bit) and leaves the other rows untouched."""
    cfg = W.SPARSE.with_(n_prefix=5003, n_steps=2)
    kp, _ = W.prefix_kv(cfg, variant=9)
    q = W.sparse_steps(cfg, variant=9)[1]["q"]
    page, k = 16, 60
    n_pages = -(-5003 // page)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    kmin = torch.empty(8, n_pages, 128, device="cuda", dtype=torch.bfloat16)
    kmax = torch.empty_like(kmin)
    fb.fb_page_meta(shape, dev_tensor(kp, "bf16"), page, kmin, kmax)
    act = np.array([0, 1, 1, 0, 0, 1, 0, 1], dtype=bool)
    act_d = torch.from_numpy(act.astype(np.uint8)).cuda()
    pages = torch.full((8, 8, k), -7, device="cuda", dtype=torch.int32)
    bound = torch.full((8, 8, n_pages), 5.0, device="cuda", dtype=torch.float64)
    fb.fb_page_select(shape, dev_tensor(q, "bf16"), kmin, kmax, n_pages, k, pages, bound=bound,
                      active=act_d)
    torch.cuda.synchronize()
    rmin, rmax = OQ.page_meta(vals(kp, "bf16"), page)
    rb = OQ.page_bound(vals(q, "bf16"), rmin, rmax)
    got_b, got_p = cpu(bound), cpu(pages)
    assert np.array_equal(got_b[act], rb[act])
    assert np.array_equal(got_p[act], OQ.topk_pages(rb, k)[act])
    assert (got_b[~act] == 5.0).all() and (got_p[~act] == -7).all()


@pytest.mark.parametrize("sel_bitmap", [True, False], ids=["bitmap_buffer", "no_bitmap_buffer"])
def test_losa_block_more_than_64_tokens(fb, sel_bitmap):
    """72 block tokens: more than a GATHER workgroup takes the union of, so
    the top-k writes page lists only and a selection prep builds the union,
    with or without a bitmap buffer in the step."""
    B = 72
    cfg = W.SPARSE.with_(n_prefix=2048, density=0.3, n_block=B, n_steps=3)
    steps = W.sparse_steps(cfg, variant=7, m_override=[None, 30, 4])
    kp, vp = W.prefix_kv(cfg, variant=7)
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    step = fb.Step(fb.FB_STEP_SPARSE, shape, B, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                   page_size=cfg.page, k_pages=cfg.k_pages, pct=cfg.pct, reselect=True,
                   sel_bitmap=sel_bitmap)
    ks = [dict(q=vals(s["q"], "bf16"), k=vals(s["k"], "bf16"), v=vals(s["v"], "bf16"))
          for s in steps]
    recs = OC.losa_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, cfg.k_pages,
                         cfg.page, cfg.pct)
    for s, (st, rec) in enumerate(zip(steps, recs)):
        a = torch.empty(B, 32, 128, device="cuda")
        l = torch.empty(B, 32, device="cuda")
        step.step(dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                  dev_tensor(st["v"], "bf16"), a, l)
        torch.cuda.synchronize()
        tag = "B72 step %d" % s
        act = rec["active"]
        if s > 0:
            assert mse_margin_ok(rec["mse"]), tag
            check_mse(tag, cpu(step.mse), rec["mse"])
        assert np.array_equal(cpu(step.active).astype(bool), act), tag
        if s > 0:
            assert np.array_equal(cpu(step.pages)[act], rec["sel"][act]), tag
        check_a(tag + " A_out", cpu(step.a_out), rec["a_out"], 2e-3)
        check_l(tag + " L_out", cpu(step.l_out), rec["l_out"], 1e-3)
        check_a(tag + " A_full", cpu(a), rec["a_full"], 2e-3)
        check_l(tag + " L_full", cpu(l), rec["l_full"], 1e-3)
