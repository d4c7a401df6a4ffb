"""GPU parity of the in-block pass + merge, the reuse decisions and the page
selector against the oracle. Masks, counts and page indices are compared bit
for bit; floats to the stated tolerance."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from oracle import quest as OQ
from oracle.attention import attn_gqa, merge
from _helpers import check_a, check_l, check_mse, cpu, dev_tensor, mse_margin_ok, tols, vals

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,n_q", [(W.TINY, 4), (W.TEXT, 4), (W.LONG, 16), (W.LONG, 1),
                                     (W.VIDEO.with_(head_dim=128), 70)],
                         ids=["tiny_f32", "text_b4", "long_b16", "b1", "mha_b70"])
def test_block_merge_matches_oracle(fb, cfg, n_q):
    cfg = cfg.with_(n_block=n_q, n_steps=1, n_prefix=600)
    st = W.text_steps(cfg)[0]
    kp, vp = W.prefix_kv(cfg)
    q, k, v = (vals(st[x], cfg.dtype) for x in ("q", "k", "v"))
    ao, lo = attn_gqa(q, vals(kp, cfg.dtype), vals(vp, cfg.dtype), cfg.scale)
    ai, li = attn_gqa(q, k, v, cfg.scale)
    af, lf = merge(ao, lo, ai, li)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, tdt)
    out = [torch.empty(n_q, cfg.n_q_heads, cfg.head_dim, device="cuda") for _ in range(2)]
    outl = [torch.empty(n_q, cfg.n_q_heads, device="cuda") for _ in range(2)]
    fb.fb_block_attn_merge(shape, dev_tensor(st["q"], cfg.dtype), dev_tensor(st["k"], cfg.dtype),
                           dev_tensor(st["v"], cfg.dtype),
                           torch.from_numpy(ao.astype(np.float32)).cuda(),
                           torch.from_numpy(lo.astype(np.float32)).cuda(),
                           out[0], outl[0], out[1], outl[1])
    torch.cuda.synchronize()
    atol, ltol = tols(cfg.dtype)
    check_a("A_in", cpu(out[1]), ai, atol)
    check_l("L_in", cpu(outl[1]), li, ltol)
    check_a("A_full", cpu(out[0]), af, atol)
    check_l("L_full", cpu(outl[0]), lf, ltol)


def test_block_merge_with_empty_cache(fb):
    cfg = W.LONG.with_(n_block=8, n_steps=1)
    st = W.text_steps(cfg)[0]
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    a_out = torch.zeros(8, 32, 128, device="cuda")
    l_out = torch.full((8, 32), float("-inf"), device="cuda")
    af = torch.empty(8, 32, 128, device="cuda")
    lf = torch.empty(8, 32, device="cuda")
    fb.fb_block_attn_merge(shape, dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                           dev_tensor(st["v"], "bf16"), a_out, l_out, af, lf)
    ai, li = attn_gqa(vals(st["q"], "bf16"), vals(st["k"], "bf16"), vals(st["v"], "bf16"), cfg.scale)
    check_a("A_full=A_in", cpu(af), ai, 2e-3)
    check_l("L_full=L_in", cpu(lf), li, 1e-3)


def _count(fb, prev, cur, tau, force, hq=32):
    args = fb.fb_reuse_args()
    args.mode = fb.FB_REUSE_COUNT
    args.n_q, args.n_heads = len(cur), hq
    p = None if prev is None else torch.tensor(prev, dtype=torch.int32, device="cuda")
    c = torch.tensor(cur, dtype=torch.int32, device="cuda")
    mask = torch.full((hq,), 9, dtype=torch.uint8, device="cuda")
    mc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    store = torch.zeros(len(cur), dtype=torch.int32, device="cuda")
    args.ids_prev, args.ids_cur = fb.ptr(p), fb.ptr(c)
    args.tau, args.force = tau, force
    args.m_count, args.ids_store, args.mask = fb.ptr(mc), fb.ptr(store), fb.ptr(mask)
    fb.fb_reuse_decide(args)
    torch.cuda.synchronize()
    return int(mc.item()), cpu(mask), cpu(store)


def test_count_bit_exact(fb):
    rng = np.random.default_rng(5)
    for trial in range(30):
        b = int(rng.integers(1, 700))
        prev = rng.integers(0, 50, b)
        cur = prev.copy()
        flip = rng.random(b) < rng.random()
        cur[flip] += 1000
        tau = int(rng.integers(0, b + 2))
        m, mask, store = _count(fb, prev, cur, tau, -1)
        want = OC.count_updated(prev, cur)
        assert m == want
        assert np.all(mask == (1 if OC.text_reuse(want, tau) else 0))
        assert np.array_equal(store, cur)
    m, mask, _ = _count(fb, None, [1, 2, 3], 2, 0)
    assert m == 3 and np.all(mask == 0)
    m, mask, _ = _count(fb, [1, 2, 3], [1, 2, 4], 0, 1)        # forced reuse
    assert m == 1 and np.all(mask == 1)


def test_head_cos_bit_exact_decisions(fb):
    rng = np.random.default_rng(11)
    nq, hq, d = 300, 12, 128
    a_c = rng.standard_normal((nq, hq, d)).astype(np.float32)
    noise = np.array([0.0, 1e-3, 0.1, 0.3, 0.33, 0.5, 1.0, 3.0, 0.2, 0.25, 0.05, 0.8])
    a_p = (a_c + noise[None, :, None] * rng.standard_normal((nq, hq, d))).astype(np.float32)
    a_p[:, 7] = 0.0                                   # one zero side -> sim 0
    mask_in = np.zeros(hq, np.uint8)
    mask_in[9] = 1                                    # reused head keeps its sim
    gamma = 0.95
    args = fb.fb_reuse_args()
    args.mode, args.n_q, args.n_heads, args.head_dim = fb.FB_REUSE_HEAD_COS, nq, hq, d
    dc, dp = torch.from_numpy(a_c).cuda(), torch.from_numpy(a_p).cuda()
    sim = torch.full((hq,), -7.0, dtype=torch.float64, device="cuda")
    mask = torch.zeros(hq, dtype=torch.uint8, device="cuda")
    mi = torch.from_numpy(mask_in).cuda()
    args.a_cached, args.a_probe, args.mask_in = dc.data_ptr(), dp.data_ptr(), mi.data_ptr()
    args.gamma, args.sim, args.mask = gamma, sim.data_ptr(), mask.data_ptr()
    ws = torch.empty(fb.fb_reuse_decide_workspace(args), dtype=torch.uint8, device="cuda")
    args.ws, args.ws_bytes = ws.data_ptr(), ws.numel()
    fb.fb_reuse_decide(args)
    torch.cuda.synchronize()
    want = OC.head_cosine(a_p, a_c)
    got = cpu(sim)
    for h in range(hq):
        if mask_in[h]:
            assert got[h] == -7.0 and cpu(mask)[h] == 1
        else:
            assert abs(got[h] - want[h]) < 1e-12
            assert cpu(mask)[h] == (1 if OC.head_reuse(want[h], gamma) else 0)
    assert got[7] == 0.0 and got[0] == 1.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_active_mse_matches_oracle(fb, dtype):
    cfg = W.SPARSE.with_(dtype=dtype, n_steps=6)
    steps = W.sparse_steps(cfg, m_override=[None, 3, 0, 8, 1, 2])
    for s in range(1, len(steps)):
        qp, qc = steps[s - 1]["q"], steps[s]["q"]
        args = fb.fb_reuse_args()
        args.mode, args.n_q, args.n_heads, args.head_dim = fb.FB_REUSE_ACTIVE_MSE, 8, 32, 128
        dp, dc = dev_tensor(qp, dtype), dev_tensor(qc, dtype)
        mse = torch.empty(8, dtype=torch.float64, device="cuda")
        act = torch.empty(8, dtype=torch.uint8, device="cuda")
        args.q_prev, args.q_cur = dp.data_ptr(), dc.data_ptr()
        args.dtype = fb.FB_BF16 if dtype == "bf16" else fb.FB_F32
        args.pct, args.mse, args.active = 25, mse.data_ptr(), act.data_ptr()
        ws = torch.empty(fb.fb_reuse_decide_workspace(args), dtype=torch.uint8, device="cuda")
        args.ws, args.ws_bytes = ws.data_ptr(), ws.numel()
        fb.fb_reuse_decide(args)
        torch.cuda.synchronize()
        want = OC.active_mse(vals(qp, dtype), vals(qc, dtype))
        assert mse_margin_ok(want), (s, want)
        check_mse("step %d" % s, cpu(mse), want)
        assert np.array_equal(cpu(act).astype(bool), OC.active_set(want, 25))


@pytest.mark.parametrize("n_kv,page,k", [(65536, 16, 819), (1000, 16, 7), (4096, 16, 0), (333, 8, 42),
                                          (100000, 16, 1875), (140000, 16, 3000)],
                         ids=["64k_d02", "ragged", "k0", "page8", "6250_pages", "8750_pages"])
def test_page_meta_and_select_bit_exact(fb, n_kv, page, k):
    cfg = W.SPARSE.with_(n_prefix=n_kv, page=page)
    kp, _ = W.prefix_kv(cfg)
    q = W.sparse_steps(cfg.with_(n_steps=1))[0]["q"]
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    n_pages = (n_kv + page - 1) // page
    kmin = torch.empty(8, n_pages, 128, dtype=torch.bfloat16, device="cuda")
    kmax = torch.empty_like(kmin)
    fb.fb_page_meta(shape, dev_tensor(kp, "bf16"), page, kmin, kmax)
    bound = torch.empty(8, 8, n_pages, dtype=torch.float64, device="cuda")
    pages = torch.full((8, 8, max(k, 1)), -1, dtype=torch.int32, device="cuda")
    fb.fb_page_select(shape, dev_tensor(q, "bf16"), kmin, kmax, n_pages, k, pages, bound=bound)
    torch.cuda.synchronize()
    rmin, rmax = OQ.page_meta(vals(kp, "bf16"), page)
    assert np.array_equal(cpu(kmin.float()), rmin) and np.array_equal(cpu(kmax.float()), rmax)
    rb = OQ.page_bound(vals(q, "bf16"), rmin, rmax)
    assert np.array_equal(cpu(bound), rb)
    if k:
        assert np.array_equal(cpu(pages), OQ.topk_pages(rb, k))


@pytest.mark.parametrize("n_take", [1, 7, 31, 32])
def test_page_select_ties_take_lower_ids(fb, n_take):
    # pages 10..40 are copies of page 5: their bounds tie exactly, and k puts
    # the selection boundary inside the tied group (taking the first, some,
    # all but one, or all of the 32 tied pages: the radix select ends on the
    # group's maximum, runs every pass, or ends on its minimum)
    n_kv, page = 4096, 16
    cfg = W.SPARSE.with_(n_prefix=n_kv, page=page)
    kp, _ = W.prefix_kv(cfg)
    kp = kp.copy()
    for pg in range(10, 41):
        kp[pg * page:(pg + 1) * page] = kp[5 * page:6 * page]
    q = W.sparse_steps(cfg.with_(n_steps=1))[0]["q"]
    rmin, rmax = OQ.page_meta(vals(kp, "bf16"), page)
    rb = OQ.page_bound(vals(q, "bf16"), rmin, rmax)
    t, g = 3, 2
    row = rb[t, g]
    above = int(np.sum(row > row[5]))
    k = above + n_take
    ref = OQ.topk_pages(rb, k)
    tied = set(range(10, 41)) | {5}
    assert len(tied & set(ref[t, g].tolist())) == n_take
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    n_pages = n_kv // page
    kmin = torch.empty(8, n_pages, 128, dtype=torch.bfloat16, device="cuda")
    kmax = torch.empty_like(kmin)
    fb.fb_page_meta(shape, dev_tensor(kp, "bf16"), page, kmin, kmax)
    pages = torch.full((8, 8, k), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(fb.fb_page_select_workspace(shape, 8, n_pages), dtype=torch.uint8, device="cuda")
    fb.fb_page_select(shape, dev_tensor(q, "bf16"), kmin, kmax, n_pages, k, pages, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(cpu(pages), ref)


@pytest.mark.parametrize("hq,hkv,dt,d", [(16, 8, "bf16", 128), (64, 8, "bf16", 128),
                                         (32, 2, "bf16", 128), (32, 8, "f32", 64),
                                         (24, 3, "f32", 128)],
                         ids=["G2", "G8", "G16_generic", "f32_G4_d64", "f32_G8_three_groups"])
def test_page_select_group_sizes(fb, hq, hkv, dt, d):
    """The bound kernel is built per group size (1, 2, 4, 8 query heads per KV
    head, bf16 and float32) with a generic form for the rest: every form gives
    the oracle's bounds and pages bit for bit."""
    n_kv, page, k = 5000, 16, 60
    cfg = W.SPARSE.with_(n_prefix=n_kv, page=page, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                         dtype=dt)
    kp, _ = W.prefix_kv(cfg)
    q = W.sparse_steps(cfg.with_(n_steps=1))[0]["q"]
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    shape = fb.shape_of(hq, hkv, d, cfg.scale, tdt)
    n_pages = (n_kv + page - 1) // page
    kmin = torch.empty(hkv, n_pages, d, dtype=tdt, device="cuda")
    kmax = torch.empty_like(kmin)
    fb.fb_page_meta(shape, dev_tensor(kp, dt), page, kmin, kmax)
    bound = torch.empty(8, hkv, n_pages, dtype=torch.float64, device="cuda")
    pages = torch.full((8, hkv, k), -1, dtype=torch.int32, device="cuda")
    fb.fb_page_select(shape, dev_tensor(q, dt), kmin, kmax, n_pages, k, pages, bound=bound)
    torch.cuda.synchronize()
    rmin, rmax = OQ.page_meta(vals(kp, dt), page)
    assert np.array_equal(cpu(kmin.float()), rmin) and np.array_equal(cpu(kmax.float()), rmax)
    rb = OQ.page_bound(vals(q, dt), rmin, rmax)
    assert np.array_equal(cpu(bound), rb)
    assert np.array_equal(cpu(pages), OQ.topk_pages(rb, k))
