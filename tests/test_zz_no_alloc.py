"""fb_prefix_attn_noalloc (the prefix pass for callers that cannot allocate:
its split-K scratch is a fixed per-device array inside the library) against
fb_prefix_attn with a caller workspace, through the C ABI: two calls in a
row, the second smaller, then a sparse GATHER call; every output bit for
bit (same kernels, same split) and within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import attn_gqa
from oracle import quest as OQ
from _helpers import check_a, check_l, cpu, dev_tensor, vals

pytestmark = pytest.mark.gpu


def _both(fb, shape, q, kd, vd, n_q, n_kv, hq, d, sel=None, a_res=None, l_res=None, a0=None,
          l0=None):
    outs = []
    for noalloc in (True, False):
        a = torch.full((n_q, hq, d), 7.0, device="cuda") if a0 is None else a0.clone()
        l = torch.full((n_q, hq), 7.0, device="cuda") if l0 is None else l0.clone()
        if noalloc:
            fb.fb_prefix_attn_noalloc(shape, q, kd, vd, a, l, sel=sel, a_res=a_res, l_res=l_res)
        else:
            nb = fb.fb_prefix_attn_workspace(shape, n_q, n_kv, sel)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
            fb.fb_prefix_attn(shape, q, kd, vd, a, l, sel=sel, a_res=a_res, l_res=l_res, ws=ws)
        torch.cuda.synchronize()
        outs.append((cpu(a), cpu(l)))
    (a1, l1), (a2, l2) = outs
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
    return a1, l1


@pytest.mark.parametrize("n_q,n_kv,layout", [(16, 200000, "head"), (8, 50000, "token")])
def test_noalloc_matches_workspace_call(fb, n_q, n_kv, layout):
    cfg = W.LONG.with_(n_prefix=n_kv, n_block=n_q)
    hq, hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    kp, vp = W.prefix_kv(cfg)
    q = W.text_steps(cfg.with_(n_steps=1))[0]["q"]
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    assert 0 < fb.fb_prefix_attn_workspace(shape, n_q, n_kv) <= fb.NOALLOC_SCRATCH_BYTES
    a, l = _both(fb, shape, dev_tensor(q, "bf16"), dev_tensor(kp, "bf16", layout),
                 dev_tensor(vp, "bf16", layout), n_q, n_kv, hq, d)
    ra, rl = attn_gqa(vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale)
    check_a("noalloc A_out", a, ra, 2e-3)
    check_l("noalloc L_out", l, rl, 1e-3)


def test_noalloc_sparse_gather(fb):
    cfg = W.SPARSE.with_(n_prefix=20000)
    hq, hkv, d, page, k = 32, 8, 128, 16, 300
    kp, vp = W.prefix_kv(cfg, variant=3)
    q = W.sparse_steps(cfg.with_(n_steps=1), variant=3)[0]["q"]
    rng = np.random.default_rng(11)
    n_pages = -(-20000 // page)
    sel = np.sort(np.stack([[rng.choice(n_pages, k, replace=False) for _ in range(hkv)]
                            for _ in range(8)]), axis=-1).astype(np.int32)
    active = np.array([1, 0, 1, 1, 0, 1, 1, 0], dtype=np.uint8)
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    pages_d = torch.from_numpy(sel).cuda()
    act_d = torch.from_numpy(active).cuda()
    s = fb.page_sel(fb.FB_SEL_GATHER, page, pages_d, act_d)
    a_res = torch.zeros(8, hq, d, device="cuda")
    l_res = torch.full((8, hq), float("-inf"), device="cuda")
    a, l = _both(fb, shape, dev_tensor(q, "bf16"), dev_tensor(kp, "bf16", "head"),
                 dev_tensor(vp, "bf16", "head"), 8, 20000, hq, d, sel=s, a_res=a_res, l_res=l_res)
    on = active.astype(bool)
    assert np.all(a[~on] == 7.0) and np.all(l[~on] == 7.0)
    (ra, rl), _ = OQ.split_attn(vals(q[on], "bf16"), vals(kp, "bf16"), vals(vp, "bf16"), sel[on],
                                page, cfg.scale, residual=False)
    check_a("noalloc gather A", a[on], ra, 2e-3)
    check_l("noalloc gather L", l[on], rl, 1e-3)
