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


def _inputs(n_q, n_kv, page, k, seed=0, hq=32, hkv=8, dtype="bf16"):
    cfg = W.SPARSE.with_(n_prefix=n_kv, n_block=n_q, n_steps=1, n_q_heads=hq, n_kv_heads=hkv,
                         dtype=dtype)
    kp, vp = W.prefix_kv(cfg)
    q = W.text_steps(cfg)[0]["q"]
    n_pages = -(-n_kv // page)
    rng = np.random.default_rng(seed)
    sel = np.stack([np.stack([np.sort(rng.choice(n_pages, size=k, replace=False))
                              for _ in range(hkv)]) for _ in range(n_q)]).astype(np.int32)
    return cfg, q, kp, vp, sel


def _bitmaps(fb, shape, pages, n_pages):
    bm = torch.full((pages.shape[0], pages.shape[1], -(-n_pages // 32)), -1, dtype=torch.int32,
                    device="cuda")
    fb.fb_page_bitmap(shape, pages, n_pages, bm)
    torch.cuda.synchronize()
    return bm


def _run(fb, cfg, q, kp, vp, sel, page, mode, active=None, a_res=None, l_res=None, a0=None, l0=None,
         prebuilt=False):
    n_q, hq, d = q.shape
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = fb.shape_of(hq, cfg.n_kv_heads, d, cfg.scale, tdt)
    pages = torch.from_numpy(sel).cuda()
    act = None if active is None else torch.from_numpy(active.astype(np.uint8)).cuda()
    bm = _bitmaps(fb, shape, pages, -(-kp.shape[0] // page)) if prebuilt else None
    s = fb.page_sel(mode, page, None if prebuilt else pages, act, bm)
    a = torch.from_numpy(a0).cuda() if a0 is not None else torch.full((n_q, hq, d), 7.0, device="cuda")
    l = torch.from_numpy(l0).cuda() if l0 is not None else torch.full((n_q, hq), 7.0, device="cuda")
    if a_res is None:
        ar = torch.full((n_q, hq, d), 7.0, device="cuda")
        lr = torch.full((n_q, hq), 7.0, device="cuda")
    else:
        ar, lr = torch.from_numpy(a_res).cuda(), torch.from_numpy(l_res).cuda()
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, n_q, kp.shape[0], s), 16),
                     dtype=torch.uint8, device="cuda")
    fb.fb_prefix_attn(shape, dev_tensor(q, cfg.dtype), dev_tensor(kp, cfg.dtype),
                      dev_tensor(vp, cfg.dtype), a, l, sel=s, a_res=ar, l_res=lr, ws=ws)
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


def test_page_bitmap_encodes_the_page_lists(fb):
    # every row's set bits are exactly its pages (ids outside [0, P) set none)
    cfg, q, kp, vp, sel = _inputs(8, 20007, 16, 300, seed=5)
    n_pages = -(-20007 // 16)
    sel = sel.copy()
    sel[0, 0, 0] = -2
    sel[1, 3, -1] = n_pages + 5
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    bm = cpu(_bitmaps(fb, shape, torch.from_numpy(sel).cuda(), n_pages)).view(np.uint32)
    for t in range(8):
        for g in range(8):
            bits = np.unpackbits(bm[t, g].view(np.uint8), bitorder="little")
            got = np.nonzero(bits)[0]
            want = np.array(sorted(p for p in sel[t, g] if 0 <= p < n_pages))
            assert np.array_equal(got, want), (t, g)


@pytest.mark.parametrize("name,n_q,n_kv,page,k,pattern", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_gather_with_prebuilt_bitmaps_is_bit_identical(fb, name, n_q, n_kv, page, k, pattern):
    """The union taken inside the GATHER workgroups from caller bitmaps gives
    the same slices, so the same partials and bit-identical outputs, as the
    selection prep's compacted union."""
    cfg, q, kp, vp, sel = _inputs(n_q, n_kv, page, k, seed=1)
    active = {"all": np.ones(n_q, bool), "mostly": np.arange(n_q) % 4 != 0,
              "one": np.arange(n_q) == 5, "none": np.zeros(n_q, bool)}[pattern]
    qv, kv, vv = vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel, page, cfg.scale)
    a_r32, l_r32 = a_r.astype(np.float32), l_r.astype(np.float32)
    a0 = np.full(a_s.shape, 7.0, np.float32)
    l0 = np.full(l_s.shape, 7.0, np.float32)
    outs = [_run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_GATHER, active=active, a_res=a_r32,
                 l_res=l_r32, a0=a0, l0=l0, prebuilt=pb) for pb in (False, True)]
    for x, y in zip(*outs):
        assert np.array_equal(x, y), name


def test_split_with_prebuilt_bitmaps_is_bit_identical(fb):
    cfg, q, kp, vp, sel = _inputs(8, 20007, 16, 250, seed=3)
    outs = [_run(fb, cfg, q, kp, vp, sel, 16, fb.FB_SEL_SPLIT, prebuilt=pb) for pb in (False, True)]
    for x, y in zip(*outs):
        assert np.array_equal(x, y)


# 128 block tokens x 32 query heads = 4,096 rows: the split-K reduce's
# many-row form (one wave per row). 2,048 keys give 2 chunks; 66,000 keys give
# 9 (the slice bound of the union), past the chunks whose partials that form
# loads up front. The oracle runs on the listed tokens only (each token has its
# own pages, so a token's rows need nothing from the others).
MANY_ROWS = [
    # name, n_q, n_kv, page, k, min chunks, tokens checked (None: all)
    ("b128_2k", 128, 2048, 16, 40, 2, None),
    ("b128_66k", 128, 66000, 16, 600, 9, (0, 3, 37, 64, 101, 127)),
]


def _chunks_at_least(fb, n_q, n_kv, page, mode, nc, per_chunk_arrays):
    shape = fb.shape_of(32, 8, 128, W.SPARSE.scale, torch.bfloat16)
    s = fb.page_sel(mode, page, torch.zeros((n_q, 8, 1), dtype=torch.int32))
    ws = fb.fb_prefix_attn_workspace(shape, n_q, n_kv, s)
    return ws >= per_chunk_arrays * nc * n_q * 32 * 128 * 4


@pytest.mark.parametrize("name,n_q,n_kv,page,k,nc,toks", MANY_ROWS, ids=[c[0] for c in MANY_ROWS])
def test_split_many_rows(fb, name, n_q, n_kv, page, k, nc, toks):
    assert _chunks_at_least(fb, n_q, n_kv, page, fb.FB_SEL_SPLIT, nc, 2)
    cfg, q, kp, vp, sel = _inputs(n_q, n_kv, page, k, seed=6)
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_SPLIT)
    t = np.arange(n_q) if toks is None else np.asarray(toks)
    qv, kv, vv = vals(q[t], "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel[t], page, cfg.scale)
    a_all, l_all = merge(a_s, l_s, a_r, l_r)
    check_a(name + " A_res", ar[t], a_r, 2e-3)
    check_l(name + " L_res", lr[t], l_r, 1e-3)
    check_a(name + " A_out", a[t], a_all, 2e-3)
    check_l(name + " L_out", l[t], l_all, 1e-3)


@pytest.mark.parametrize("name,n_q,n_kv,page,k,nc,toks", MANY_ROWS, ids=[c[0] for c in MANY_ROWS])
def test_gather_many_rows(fb, name, n_q, n_kv, page, k, nc, toks):
    assert _chunks_at_least(fb, n_q, n_kv, page, fb.FB_SEL_GATHER, nc, 1)
    cfg, q, kp, vp, sel = _inputs(n_q, n_kv, page, k, seed=7)
    active = np.arange(n_q) % 4 != 1
    t = np.arange(n_q) if toks is None else np.asarray(toks)
    qv, kv, vv = vals(q[t], "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel[t], page, cfg.scale)
    # cached residual: the oracle's for the checked tokens, seeded values for the rest
    rng = np.random.default_rng(8)
    a_r32 = rng.normal(0.0, 0.05, (n_q, 32, 128)).astype(np.float32)
    l_r32 = rng.uniform(5.0, 9.0, (n_q, 32)).astype(np.float32)
    a_r32[t], l_r32[t] = a_r, l_r
    a0 = np.full((n_q, 32, 128), 7.0, np.float32)
    l0 = np.full((n_q, 32), 7.0, np.float32)
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_GATHER, active=active,
                        a_res=a_r32, l_res=l_r32, a0=a0, l0=l0)
    ref_a, ref_l = merge(a_s, l_s, a_r32[t].astype(np.float64), l_r32[t].astype(np.float64))
    assert np.all(a[~active] == 7.0) and np.all(l[~active] == 7.0)
    on = active[t]
    check_a(name + " A_out", a[t][on], ref_a[on], 2e-3)
    check_l(name + " L_out", l[t][on], ref_l[on], 1e-3)
    assert np.array_equal(ar, a_r32) and np.array_equal(lr, l_r32)   # inputs untouched
    # caller-built bitmaps (their union from its own launch at this many tokens)
    pb = _run(fb, cfg, q, kp, vp, sel, page, fb.FB_SEL_GATHER, active=active, a_res=a_r32,
              l_res=l_r32, a0=a0, l0=l0, prebuilt=True)
    for x, y in zip((a, l, ar, lr), pb):
        assert np.array_equal(x, y), name


@pytest.mark.parametrize("n_q", [64, 65])
def test_gather_prebuilt_at_the_token_bound(fb, n_q):
    """Up to 64 tokens a GATHER workgroup takes the union of the caller's
    bitmaps itself, from 65 on a launch of its own builds it: both give the
    oracle's pairs and the prep path's bits."""
    cfg, q, kp, vp, sel = _inputs(n_q, 3000, 16, 40, seed=10)
    active = np.arange(n_q) % 3 != 2
    qv, kv, vv = vals(q, "bf16"), vals(kp, "bf16"), vals(vp, "bf16")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel, 16, cfg.scale)
    a_r32, l_r32 = a_r.astype(np.float32), l_r.astype(np.float32)
    a0 = np.full(a_s.shape, 7.0, np.float32)
    l0 = np.full(l_s.shape, 7.0, np.float32)
    outs = [_run(fb, cfg, q, kp, vp, sel, 16, fb.FB_SEL_GATHER, active=active, a_res=a_r32,
                 l_res=l_r32, a0=a0, l0=l0, prebuilt=pb) for pb in (True, False)]
    a, l = outs[0][0], outs[0][1]
    ref_a, ref_l = merge(a_s, l_s, a_r32.astype(np.float64), l_r32.astype(np.float64))
    assert np.all(a[~active] == 7.0) and np.all(l[~active] == 7.0)
    check_a("n_q %d A_out" % n_q, a[active], ref_a[active], 2e-3)
    check_l("n_q %d L_out" % n_q, l[active], ref_l[active], 1e-3)
    for x, y in zip(*outs):
        assert np.array_equal(x, y), n_q


def test_split_many_rows_f32(fb):
    """float32 K/V (the generic kernel, one chunk) at 4,096 rows: its partials
    through the many-row reduce, residual included."""
    cfg, q, kp, vp, sel = _inputs(128, 1500, 16, 30, seed=9, dtype="f32")
    a, l, ar, lr = _run(fb, cfg, q, kp, vp, sel, 16, fb.FB_SEL_SPLIT)
    qv, kv, vv = vals(q, "f32"), vals(kp, "f32"), vals(vp, "f32")
    (a_s, l_s), (a_r, l_r) = split_attn(qv, kv, vv, sel, 16, cfg.scale)
    a_all, l_all = merge(a_s, l_s, a_r, l_r)
    check_a("f32 A_res", ar, a_r, 1e-5)
    check_l("f32 L_res", lr, l_r, 1e-5)
    check_a("f32 A_out", a, a_all, 1e-5)
    check_l("f32 L_out", l, l_all, 1e-5)
