"""GPU parity of the many-rows MFMA path against the oracle.

A pass runs on this path when a KV head serves >= 128 query rows (bf16,
d = 128): the prefill regime of video generation (thousands of block queries
per head) and large text blocks. Cases span several row tiles with a ragged
last tile, ragged key tiles, split-K chunks, head-major K/V, grouped-query
heads, masked heads, and the in-block pass with the merge in its epilogue.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle.attention import attn_gqa, merge
from _helpers import check_a, check_l, cpu, dev_tensor, run_prefix, tols, vals

pytestmark = pytest.mark.gpu

PREFIX_CASES = [
    # name, cfg, n_q, n_kv, layout
    ("mha_300x1000", W.VIDEO, 300, 1000, "tok"),          # 3 row tiles, ragged keys, direct
    ("mha_300x9000_splitk", W.VIDEO, 300, 9000, "tok"),   # split-K partials + reduce
    ("mha_350x9000_lean_reduce", W.VIDEO, 350, 9000, "tok"),  # 4200 rows: many-row reduce
    ("mha_200x2500_headmajor", W.VIDEO, 200, 2500, "head"),
    ("gqa_50x5000", W.LONG, 50, 5000, "tok"),             # 200 rows per KV head
    ("gqa_64x33", W.LONG, 64, 33, "tok"),                 # last key tile holds one key
    ("mha_129x1", W.VIDEO, 129, 1, "tok"),                # a single key
]


def _plan_is_split(fb, cfg, n_q, n_kv):
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, torch.bfloat16)
    return fb.fb_prefix_attn_workspace(shape, n_q, n_kv) > 0


@pytest.mark.parametrize("name,cfg,n_q,n_kv,layout", PREFIX_CASES, ids=[c[0] for c in PREFIX_CASES])
def test_rows_prefix_matches_oracle(fb, name, cfg, n_q, n_kv, layout):
    a, l, ra, rl, cfg = run_prefix(fb, cfg, n_q, n_kv, layout)
    atol, ltol = tols(cfg.dtype)
    check_a(name + " A_out", a, ra, atol)
    check_l(name + " L_out", l, rl, ltol)


def test_rows_split_plan_is_exercised(fb):
    assert _plan_is_split(fb, W.VIDEO, 300, 9000)
    assert _plan_is_split(fb, W.VIDEO, 350, 9000)
    assert not _plan_is_split(fb, W.VIDEO, 300, 1000)


@pytest.mark.parametrize("gain", [2.0, 4.0])
def test_rows_prefix_peaked(fb, gain):
    a, l, ra, rl, cfg = run_prefix(fb, W.VIDEO, 256, 3000, q_gain=gain)
    check_a("peaked A_out", a, ra, 2e-3)
    check_l("peaked L_out", l, rl, 1e-3)


def test_rows_prefix_masked_heads_untouched(fb):
    mask = [0] * 12
    for h in (0, 5, 11):
        mask[h] = 1
    a, l, ra, rl, cfg = run_prefix(fb, W.VIDEO, 260, 2000, mask=mask)
    m = np.array(mask, bool)
    assert np.all(a[:, m] == 7.0) and np.all(l[:, m] == 7.0)
    check_a("unmasked A_out", a[:, ~m], ra[:, ~m], 2e-3)
    check_l("unmasked L_out", l[:, ~m], rl[:, ~m], 1e-3)


def test_rows_prefix_deterministic(fb):
    a1, l1, *_ = run_prefix(fb, W.VIDEO, 300, 9000)
    a2, l2, *_ = run_prefix(fb, W.VIDEO, 300, 9000)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)


BLOCK_CASES = [
    ("mha_300", W.VIDEO, 300),
    ("mha_128", W.VIDEO, 128),
    ("gqa_40", W.LONG, 40),          # 160 rows per KV head
    ("gqa_33", W.LONG, 33),          # 132 rows: one full tile and a 4-row tail
]


@pytest.mark.parametrize("name,cfg,n_q", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_rows_block_merge_matches_oracle(fb, name, cfg, n_q):
    cfg = cfg.with_(n_block=n_q, n_steps=1, n_prefix=700)
    st = W.text_steps(cfg)[0]
    kp, vp = W.prefix_kv(cfg)
    q, k, v = (vals(st[x], "bf16") for x in ("q", "k", "v"))
    ao, lo = attn_gqa(q, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale)
    lo[::7, ::3] = -np.inf                     # some rows without a cached side
    ao[::7, ::3] = 0.0
    ai, li = attn_gqa(q, k, v, cfg.scale)
    af, lf = merge(ao, lo, ai, li)
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, 128, cfg.scale, torch.bfloat16)
    hq = cfg.n_q_heads
    out = [torch.empty(n_q, hq, 128, device="cuda") for _ in range(2)]
    outl = [torch.empty(n_q, hq, device="cuda") for _ in range(2)]
    fb.fb_block_attn_merge(shape, dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                           dev_tensor(st["v"], "bf16"),
                           torch.from_numpy(ao.astype(np.float32)).cuda(),
                           torch.from_numpy(lo.astype(np.float32)).cuda(),
                           out[0], outl[0], out[1], outl[1])
    torch.cuda.synchronize()
    check_a(name + " A_in", cpu(out[1]), ai, 2e-3)
    check_l(name + " L_in", cpu(outl[1]), li, 1e-3)
    check_a(name + " A_full", cpu(out[0]), af, 2e-3)
    check_l(name + " L_full", cpu(outl[0]), lf, 1e-3)


def test_rows_block_merge_optional_outputs(fb):
    # l_full, a_in and l_in are optional: A_full alone must match
    cfg = W.VIDEO.with_(n_block=200, n_steps=1)
    st = W.text_steps(cfg)[0]
    q, k, v = (vals(st[x], "bf16") for x in ("q", "k", "v"))
    ai, li = attn_gqa(q, k, v, cfg.scale)
    rng = np.random.default_rng(5)
    ao = rng.standard_normal((200, 12, 128)).astype(np.float32) * 0.05
    lo = (rng.standard_normal((200, 12)) + 6.0).astype(np.float32)
    af, _ = merge(ao.astype(np.float64), lo.astype(np.float64), ai, li)
    shape = fb.shape_of(12, 12, 128, cfg.scale, torch.bfloat16)
    a = torch.empty(200, 12, 128, device="cuda")
    fb.fb_block_attn_merge(shape, dev_tensor(st["q"], "bf16"), dev_tensor(st["k"], "bf16"),
                           dev_tensor(st["v"], "bf16"), torch.from_numpy(ao).cuda(),
                           torch.from_numpy(lo).cuda(), a)
    torch.cuda.synchronize()
    check_a("A_full only", cpu(a), af, 2e-3)


@pytest.mark.parametrize("n_on", [1, 4, 11])
def test_rows_prefix_mask_sized_split(fb, n_on):
    # with a head mask the pass splits the keys by the number of heads left
    # (partials + reduce); skipped heads stay untouched
    rng = np.random.default_rng(n_on)
    on = rng.choice(12, size=n_on, replace=False)
    mask = [0 if h in on else 1 for h in range(12)]
    a, l, ra, rl, cfg = run_prefix(fb, W.VIDEO, 300, 9000, mask=mask)
    m = np.array(mask, bool)
    assert np.all(a[:, m] == 7.0) and np.all(l[:, m] == 7.0)
    check_a("A_out of computed heads", a[:, ~m], ra[:, ~m], 2e-3)
    check_l("L_out of computed heads", l[:, ~m], rl[:, ~m], 1e-3)


def test_rows_prefix_very_peaked(fb):
    # Q x 8: a few keys carry almost all of each row's weight, where the
    # rounding of the weights in P.V matters most
    a, l, ra, rl, cfg = run_prefix(fb, W.VIDEO, 256, 3000, q_gain=8.0)
    check_a("very peaked A_out", a, ra, 2e-3)
    check_l("very peaked L_out", l, rl, 1e-3)



def _bf16_bits(x):
    return np.array([x], np.float32).view(np.uint32)[0] >> 16


def test_rows_prefix_large_v_entries(fb):
    # a few V entries of magnitude 1000 dominate some outputs (|A| ~ 11): the
    # hi + lo weights keep the absolute error within the output bound (one
    # bf16 or fp16 weight would not: 2^-9 or 2^-11 of ~11)
    def edit(vp):
        vp[1234, 3, 9] = _bf16_bits(1000.0)
        vp[77, 8, 64] = _bf16_bits(-1000.0)
    a, l, ra, rl, cfg = run_prefix(fb, W.VIDEO, 300, 2000, v_edit=edit)
    assert np.abs(ra).max() > 5.0
    check_a("A_out with large V entries", a, ra, 2e-3)
    check_l("L_out with large V entries", l, rl, 1e-3)
