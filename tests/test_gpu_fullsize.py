"""GPU parity at full sizes on sampled outputs, for the calls the
element-by-element bench-size tests (test_gpu_benchsize.py) do not drive:

* long-context text: the 800,000-token prefix in a growing head-major cache,
  the next block after the first one joined it;
* video: 12 MHA heads, 4,680 block queries, 12,480 prefix tokens: the prefix
  pass (plain and with a head mask) and the in-block pass with the merge
  called on their own (A_in, L_in included), and the per-head cosine
  decision on synthetic [4680, 12, 128] outputs.

The oracle computes the sampled rows one by one (float64 dense softmax over
every key of the row's KV head); properties that hold at any size (finite
outputs, untouched skipped heads) are checked on all rows.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import controller as OC
from oracle.attention import attn, merge
from _helpers import check_a, check_l, cpu, dev_tensor, vals

pytestmark = pytest.mark.gpu

N_TEXT, B_TEXT = 800000, 16


@pytest.fixture(scope="module")
def text_800k():
    cfg = W.LONG.with_(n_prefix=N_TEXT, n_block=B_TEXT)
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    return cfg, kp, vp, steps


def _rows_ref(q, kp, vp, scale, rows, hq, hkv):
    """Oracle A, L for sampled (t, h) rows; one KV head in float64 at a time."""
    G = hq // hkv
    out_a, out_l = {}, {}
    for g in sorted({h // G for _, h in rows}):
        kg = vals(kp[:, g, :], "bf16")
        vg = vals(vp[:, g, :], "bf16")
        for t, h in rows:
            if h // G != g:
                continue
            a, l = attn(vals(q[t:t + 1, h, :], "bf16"), kg, vg, scale)
            out_a[(t, h)], out_l[(t, h)] = a[0], l[0]
    return out_a, out_l


def _sample_rows(n_q, hq, n, seed):
    rng = np.random.default_rng(seed)
    return sorted({(int(rng.integers(n_q)), int(rng.integers(hq))) for _ in range(n)})


def test_text_800k_growing_cache_sampled(fb, text_800k):
    """The 800,000-token prefix in a head-major cache with room for two more
    blocks: block 0's last-step K/V are appended (bit for bit), then block 1's
    first step attends over all 800,016 cache tokens and its own 16."""
    cfg, kp, vp, steps = text_800k
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    cache = fb.KVCache(N_TEXT + 2 * B_TEXT, hkv, d, torch.bfloat16, "cuda", "head")
    cache.append(shape, dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"))
    step = fb.Step(fb.FB_STEP_TEXT, shape, B_TEXT, cache=cache, tau=cfg.tau)
    a = torch.empty(B_TEXT, hq, d, device="cuda")
    l = torch.empty(B_TEXT, hq, device="cuda")
    st0, last = steps[0], steps[-1]
    step.step(dev_tensor(st0["q"], "bf16"), dev_tensor(st0["k"], "bf16"),
              dev_tensor(st0["v"], "bf16"), a, l, ids=torch.from_numpy(st0["ids"]).cuda())
    step.next_block(dev_tensor(last["k"], "bf16"), dev_tensor(last["v"], "bf16"))
    torch.cuda.synchronize()
    assert cache.n_tok == N_TEXT + B_TEXT and step.state.step == 0
    for got, want in ((cache.k_all, last["k"]), (cache.v_all, last["v"])):
        tail = got[N_TEXT:N_TEXT + B_TEXT].cpu().contiguous().view(torch.int16).numpy()
        assert np.array_equal(tail, np.ascontiguousarray(want).view(np.int16))
    st1 = W.text_steps(cfg, block=1)[0]
    step.step(dev_tensor(st1["q"], "bf16"), dev_tensor(st1["k"], "bf16"),
              dev_tensor(st1["v"], "bf16"), a, l, ids=torch.from_numpy(st1["ids"]).cuda())
    torch.cuda.synchronize()
    a_np, l_np = cpu(a), cpu(l)
    assert np.all(np.isfinite(a_np)) and np.all(np.isfinite(l_np))
    G = hq // hkv
    rows = [(t, h) for t, h in _sample_rows(B_TEXT, hq, 40, seed=4) if h // G in (1, 6)][:10]
    for g in sorted({h // G for _, h in rows}):
        keys = np.concatenate([vals(x[:, g, :], "bf16") for x in (kp, last["k"], st1["k"])])
        vs = np.concatenate([vals(x[:, g, :], "bf16") for x in (vp, last["v"], st1["v"])])
        for t, h in rows:
            if h // G != g:
                continue
            ar, lr = attn(vals(st1["q"][t:t + 1, h, :], "bf16"), keys, vs, cfg.scale)
            check_a("grown 800k row %s A_full" % ((t, h),), a_np[t, h], ar[0], 2e-3)
            check_l("grown 800k row %s L_full" % ((t, h),), l_np[t, h:h + 1], lr, 1e-3)


@pytest.fixture(scope="module")
def video_full():
    cfg = W.VIDEO
    kp, vp = W.prefix_kv(cfg)
    st = W.video_steps(cfg.with_(n_steps=1), W.video_sigmas(cfg, 0))[0]
    return cfg, kp, vp, st


def test_video_full_prefix_and_block_sampled(fb, video_full):
    cfg, kp, vp, st = video_full
    H, d, NQ, NK = cfg.n_q_heads, cfg.head_dim, cfg.n_block, cfg.n_prefix
    shape = fb.shape_of(H, H, d, cfg.scale, torch.bfloat16)
    q, kb, vb = (dev_tensor(st[x], "bf16") for x in ("q", "k", "v"))
    kd, vd = dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16")
    a = torch.empty(NQ, H, d, device="cuda")
    l = torch.empty(NQ, H, device="cuda")
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, NQ, NK), 16), dtype=torch.uint8,
                     device="cuda")
    fb.fb_prefix_attn(shape, q, kd, vd, a, l, ws=ws)
    af = torch.empty(NQ, H, d, device="cuda")
    lf = torch.empty(NQ, H, device="cuda")
    ai = torch.empty(NQ, H, d, device="cuda")
    li = torch.empty(NQ, H, device="cuda")
    fb.fb_block_attn_merge(shape, q, kb, vb, a, l, af, lf, ai, li)
    torch.cuda.synchronize()
    A, L, AF, LF, AI, LI = (cpu(x) for x in (a, l, af, lf, ai, li))
    for x in (A, L, AF, LF):
        assert np.all(np.isfinite(x))
    rows = _sample_rows(NQ, H, 40, seed=3) + [(0, 0), (NQ - 1, H - 1)]
    for t, h in rows:
        qr = vals(st["q"][t:t + 1, h, :], "bf16")
        ao, lo = attn(qr, vals(kp[:, h, :], "bf16"), vals(vp[:, h, :], "bf16"), cfg.scale)
        ain, lin = attn(qr, vals(st["k"][:, h, :], "bf16"), vals(st["v"][:, h, :], "bf16"), cfg.scale)
        afr, lfr = merge(ao, lo, ain, lin)
        check_a("video row %s A_out" % ((t, h),), A[t, h], ao[0], 2e-3)
        check_l("video row %s L_out" % ((t, h),), L[t, h:h + 1], lo, 1e-3)
        check_a("video row %s A_in" % ((t, h),), AI[t, h], ain[0], 2e-3)
        check_l("video row %s L_in" % ((t, h),), LI[t, h:h + 1], lin, 1e-3)
        check_a("video row %s A_full" % ((t, h),), AF[t, h], afr[0], 2e-3)
        check_l("video row %s L_full" % ((t, h),), LF[t, h:h + 1], lfr, 1e-3)


def test_video_full_masked_prefix_sampled(fb, video_full):
    # 4 of 12 heads recompute: the pass splits its keys by the heads left
    cfg, kp, vp, st = video_full
    H, d, NQ, NK = cfg.n_q_heads, cfg.head_dim, cfg.n_block, cfg.n_prefix
    mask = np.ones(H, np.uint8)
    mask[[1, 4, 7, 11]] = 0
    shape = fb.shape_of(H, H, d, cfg.scale, torch.bfloat16)
    a = torch.full((NQ, H, d), 7.0, device="cuda")
    l = torch.full((NQ, H), 7.0, device="cuda")
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, NQ, NK), 16), dtype=torch.uint8,
                     device="cuda")
    fb.fb_prefix_attn(shape, dev_tensor(st["q"], "bf16"), dev_tensor(kp, "bf16"),
                      dev_tensor(vp, "bf16"), a, l, mask=torch.from_numpy(mask).cuda(), ws=ws)
    torch.cuda.synchronize()
    A, L = cpu(a), cpu(l)
    m = mask.astype(bool)
    assert np.all(A[:, m] == 7.0) and np.all(L[:, m] == 7.0)
    rows = [(t, h) for t, h in _sample_rows(NQ, H, 60, seed=4) if not m[h]]
    for t, h in rows:
        qr = vals(st["q"][t:t + 1, h, :], "bf16")
        ao, lo = attn(qr, vals(kp[:, h, :], "bf16"), vals(vp[:, h, :], "bf16"), cfg.scale)
        check_a("masked video row %s A_out" % ((t, h),), A[t, h], ao[0], 2e-3)
        check_l("masked video row %s L_out" % ((t, h),), L[t, h:h + 1], lo, 1e-3)


def test_video_full_head_cosine(fb):
    # the per-head decision at the video output size, on synthetic fp32 outputs
    rng = np.random.default_rng(21)
    nq, hq, d = 4680, 12, 128
    a_c = (0.05 * rng.standard_normal((nq, hq, d))).astype(np.float32)
    noise = np.array([0.0, 1e-3, 0.02, 0.1, 0.3, 0.5, 1.0, 2.0, 0.25, 0.33, 0.05, 0.8])
    a_p = (a_c + 0.05 * noise[None, :, None] * rng.standard_normal((nq, hq, d))).astype(np.float32)
    gamma = 0.95
    want = OC.head_cosine(a_p, a_c)
    assert np.all(np.abs(want - gamma) > 1e-6)          # no decision within rounding of gamma
    args = fb.fb_reuse_args()
    args.mode, args.n_q, args.n_heads, args.head_dim = fb.FB_REUSE_HEAD_COS, nq, hq, d
    dc, dp = torch.from_numpy(a_c).cuda(), torch.from_numpy(a_p).cuda()
    sim = torch.full((hq,), -7.0, dtype=torch.float64, device="cuda")
    mask = torch.zeros(hq, dtype=torch.uint8, device="cuda")
    args.a_cached, args.a_probe = dc.data_ptr(), dp.data_ptr()
    args.gamma, args.sim, args.mask = gamma, sim.data_ptr(), mask.data_ptr()
    ws = torch.empty(fb.fb_reuse_decide_workspace(args), dtype=torch.uint8, device="cuda")
    args.ws, args.ws_bytes = ws.data_ptr(), ws.numel()
    fb.fb_reuse_decide(args)
    torch.cuda.synchronize()
    assert np.max(np.abs(cpu(sim) - want)) < 1e-12
    assert np.array_equal(cpu(mask).astype(bool), OC.head_reuse(want, gamma))
