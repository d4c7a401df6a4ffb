"""GPU parity of the sparse block-external pass (fb_prefix_attn with a page
selection) against the oracle's split attention.

SPLIT (refresh step) must return the pair over all keys and the residual
pair over the keys outside each row's selected pages; GATHER (later steps)
must merge the pair over the selected pages with a cached residual for the
active rows and leave the other rows untouched. Selections are seeded random
page sets (the selector itself is tested elsewhere), so every row of a group
selects different pages and the union covers most of the prefix.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import merge
from oracle.quest import split_attn, union_size
from _helpers import check_a, check_l, cpu, dev_tensor, vals

pytestmark = pytest.mark.gpu


def _inputs(n_q, n_kv, page, k, seed=0, hq=32, hkv=8):
    cfg = W.SPARSE.with_(n_prefix=n_kv, n_block=n_q, n_steps=1, n_q_heads=hq, n_kv_heads=hkv)
    kp, vp = W.prefix_kv(cfg)
    q = W.text_steps(cfg)[0]["q"]
    n_pages = -(-n_kv // page)
    rng = np.random.default_rng(seed)
    sel = np.stack([np.stack([np.sort(rng.choice(n_pages, size=k, replace=False))
                              for _ in range(hkv)]) for _ in range(n_q)]).astype(np.int32)
    return cfg, q, kp, vp, sel


def _run(fb, cfg, q, kp, vp, sel, page, mode, active=None, a_res=None, l_res=None, a0=None, l0=None):
    n_q, hq, d = q.shape
    shape = fb.shape_of(hq, cfg.n_kv_heads, d, cfg.scale, torch.bfloat16)
    pages = torch.from_numpy(sel).cuda()
    act = None if active is None else torch.from_numpy(active.astype(np.uint8)).cuda()
    s = fb.page_sel(mode, page, pages, act)
    a = torch.from_numpy(a0).cuda() if a0 is not None else torch.full((n_q, hq, d), 7.0, device="cuda")
    l = torch.from_numpy(l0).cuda() if l0 is not None else torch.full((n_q, hq), 7.0, device="cuda")
    if a_res is None:
        ar = torch.full((n_q, hq, d), 7.0, device="cuda")
        lr = torch.full((n_q, hq), 7.0, device="cuda")
    else:
        ar, lr = torch.from_numpy(a_res).cuda(), torch.from_numpy(l_res).cuda()
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, n_q, kp.shape[0], s), 16),
                     dtype=torch.uint8, device="cuda")
    fb.fb_prefix_attn(shape, dev_tensor(q, "bf16"), dev_tensor(kp, "bf16"), dev_tensor(vp, "bf16"),
                      a, l, sel=s, a_res=ar, l_res=lr, ws=ws)
    torch.cuda.synchronize()
    return cpu(a), cpu(l), cpu(ar), cpu(lr)


SPLIT_CASES = [
    # name, n_q, n_kv, page, k
    ("b8_64k_d02", 8, 65536, 16, 819),
    ("b8_ragged_last_page", 8, 20007, 16, 250),
    ("b4_page32", 4, 9000, 32, 60),
    ("b3_rows12", 3, 5000, 16, 100),
    ("b8_k1", 8, 4096, 16, 1),
    ("b8_all_pages", 8, 2048, 16, 128),
]


@pytest.mark.parametrize("name,n_q,n_kv,page,k", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_matches_oracle(fb, name, n_q, n_kv, page, k):
    cfg, q, kp, vp, sel = _inputs(n_q, n_kv, page, k)
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_SPLIT)
    qv, kv, vv = vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel, page, cfg.scale)
    a_all, l_all = merge(a_s, l_s, a_r, l_r)
    check_a(name + " A_res", ar, a_r, 2e-3)
    check_l(name + " L_res", lr, l_r, 1e-3)
    check_a(name + " A_out", a, a_all, 2e-3)
    check_l(name + " L_out", l, l_all, 1e-3)


def test_split_empty_selection(fb):
    cfg, q, kp, vp, sel = _inputs(8, 3000, 16, 0)
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, 16, fb.FB_SEL_SPLIT)
    from oracle.attention import attn_gqa
    ra, rl = attn_gqa(vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale)
    check_a("all residual", ar, ra, 2e-3)
    check_l("all residual L", lr, rl, 1e-3)
    check_a("A_out", a, ra, 2e-3)


GATHER_CASES = [
    # name, n_q, n_kv, page, k, active pattern
    ("b8_64k_d02", 8, 65536, 16, 819, "mostly"),
    ("b8_64k_d04", 8, 65536, 16, 1638, "all"),
    ("b8_ragged_page32", 8, 20007, 32, 200, "mostly"),
    ("b8_one_active", 8, 30000, 16, 300, "one"),
    ("b8_none_active", 8, 4000, 16, 50, "none"),
]


@pytest.mark.parametrize("name,n_q,n_kv,page,k,pattern", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_gather_matches_oracle(fb, name, n_q, n_kv, page, k, pattern):
    cfg, q, kp, vp, sel = _inputs(n_q, n_kv, page, k, seed=1)
    active = {"all": np.ones(n_q, bool), "mostly": np.arange(n_q) % 4 != 0,
              "one": np.arange(n_q) == 5, "none": np.zeros(n_q, bool)}[pattern]
    qv, kv, vv = vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel, page, cfg.scale)
    # the cached residual as the refresh step left it (fp32)
    a_r32, l_r32 = a_r.astype(np.float32), l_r.astype(np.float32)
    a0 = np.full(a_s.shape, 7.0, np.float32)
    l0 = np.full(l_s.shape, 7.0, np.float32)
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_GATHER, active=active,
                        a_res=a_r32, l_res=l_r32, a0=a0, l0=l0)
    ref_a, ref_l = merge(a_s, l_s, a_r32.astype(np.float64), l_r32.astype(np.float64))
    assert np.all(a[~active] == 7.0) and np.all(l[~active] == 7.0)
    if active.any():
        check_a(name + " A_out", a[active], ref_a[active], 2e-3)
        check_l(name + " L_out", l[active], ref_l[active], 1e-3)
    assert np.array_equal(ar, a_r32) and np.array_equal(lr, l_r32)   # inputs untouched
    if pattern == "mostly":                   # the union really spans most of the prefix
        assert union_size(sel, active).min() > 0.5 * (-(-n_kv // page))


def test_out_of_range_page_ids_select_nothing(fb):
    cfg, q, kp, vp, sel = _inputs(8, 5000, 16, 40, seed=2)
    n_pages = -(-5000 // 16)
    bad = sel.copy()
    bad[:, :, 0] = -3                         # first id of every row out of range
    bad[:, :, -1] = n_pages + 7               # and the last
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, bad, 16, fb.FB_SEL_SPLIT)
    good = [sorted(p for p in row if 0 <= p < n_pages) for row in bad.reshape(-1, 40)]
    qv, kv, vv = vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    sel_ok = np.array(good, dtype=np.int32).reshape(8, 8, 38)
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel_ok, 16, cfg.scale)
    check_a("residual with ignored ids", ar, a_r, 2e-3)
    check_l("residual L with ignored ids", lr, l_r, 1e-3)
