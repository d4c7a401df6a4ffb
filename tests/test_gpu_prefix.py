"""GPU parity of the block-external pass (fb_prefix_attn) against the oracle.

Sizes span several split-K chunks and 32-token tiles with ragged tails; both
the MFMA decode kernel (bf16, d 128) and the generic kernel (fp32 / d 64)
are exercised, in token-major and head-major K/V layouts.
"""

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import check_a, check_l, cpu, dev_tensor, run_prefix, tols

pytestmark = pytest.mark.gpu


CASES = [
    # name, cfg, n_q, n_kv, layout
    ("tiny_f32", W.TINY, 4, 1024, "tok"),
    ("tiny_f32_ragged", W.TINY, 3, 777, "head"),
    ("text_b4_32k", W.TEXT, 4, 32768, "tok"),
    ("text_b4_32k_headmajor", W.TEXT, 4, 32768, "head"),
    ("b8_ragged", W.LONG, 8, 20001, "tok"),
    ("b16_ragged", W.LONG, 16, 20001, "tok"),
    ("b16_headmajor", W.LONG, 16, 50000, "head"),
    ("b16_two_tiles_ragged", W.LONG, 16, 33, "tok"),      # second tile holds one key
    ("b12_rows48_headmajor", W.LONG, 12, 5003, "head"),
    ("b1_short", W.LONG, 1, 45, "tok"),
    ("b32_two_slabs", W.LONG, 32, 3000, "tok"),
    ("b5_rows20", W.LONG, 5, 4096, "tok"),
    ("b5_rows20_headmajor", W.LONG, 5, 4099, "head"),  # pair kernel, one row block idle
    ("b1_short_headmajor", W.LONG, 1, 45, "head"),
    ("mha_d128_video_like", W.VIDEO, 6, 1000, "tok"),
    ("d64_bf16_generic", W.LONG.with_(head_dim=64), 4, 2000, "tok"),
]


@pytest.mark.parametrize("name,cfg,n_q,n_kv,layout", CASES, ids=[c[0] for c in CASES])
def test_prefix_matches_oracle(fb, name, cfg, n_q, n_kv, layout):
    a, l, ra, rl, cfg = run_prefix(fb, cfg, n_q, n_kv, layout)
    atol, ltol = tols(cfg.dtype)
    check_a(name + " A_out", a, ra, atol)
    check_l(name + " L_out", l, rl, ltol)


HEAD_SHAPES = [
    # name, query heads, KV heads, block tokens, layout
    ("q64_kv8_b16", 64, 8, 16, "tok"),       # 128 rows per KV head: the many-rows kernel
    ("q64_kv8_b6", 64, 8, 6, "head"),        # 48 rows: the pair kernel
    ("q28_kv4_b16", 28, 4, 16, "tok"),       # 7 query heads per KV head, two row slabs
    ("q28_kv4_b3_head", 28, 4, 3, "head"),
    ("q32_kv1_b16", 32, 1, 16, "tok"),       # one KV head: 512 rows, many-rows kernel
    ("q32_kv1_b2", 32, 1, 2, "head"),
    ("q40_kv5_b8", 40, 5, 8, "tok"),         # KV heads not a multiple of the 8 XCDs
    ("q16_kv2_b4_head", 16, 2, 4, "head"),
    ("q8_kv8_b30", 8, 8, 30, "tok"),         # one query head per KV head, 30 rows
]


@pytest.mark.parametrize("name,hq,hkv,n_q,layout", HEAD_SHAPES, ids=[c[0] for c in HEAD_SHAPES])
def test_prefix_head_shapes(fb, name, hq, hkv, n_q, layout):
    cfg = W.LONG.with_(n_q_heads=hq, n_kv_heads=hkv)
    a, l, ra, rl, cfg = run_prefix(fb, cfg, n_q, 10007, layout)
    check_a(name + " A_out", a, ra, 2e-3)
    check_l(name + " L_out", l, rl, 1e-3)


@pytest.mark.parametrize("gain", [4.0, 8.0])
def test_prefix_peaked_scores(fb, gain):
    # Q scaled up: O(1) outputs dominated by few keys, exercising the running
    # max rescale and the bf16 rounding of the softmax weights.
    a, l, ra, rl, cfg = run_prefix(fb, W.LONG, 16, 30000, q_gain=gain)
    check_a("peaked A_out", a, ra, 2e-3)
    check_l("peaked L_out", l, rl, 1e-3)
    assert np.max(np.abs(ra)) > 0.3        # the case really is peaked


def test_prefix_masked_heads_untouched(fb):
    mask = [0] * 32
    for h in (4, 5, 6, 7, 13, 31):           # group 1 fully masked, 13 and 31 alone
        mask[h] = 1
    a, l, ra, rl, cfg = run_prefix(fb, W.LONG, 8, 5000, mask=mask)
    m = np.array(mask, bool)
    assert np.all(a[:, m] == 7.0) and np.all(l[:, m] == 7.0)
    check_a("unmasked A_out", a[:, ~m], ra[:, ~m], 2e-3)
    check_l("unmasked L_out", l[:, ~m], rl[:, ~m], 1e-3)


def test_prefix_empty_prefix(fb):
    cfg = W.LONG
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    q = dev_tensor(W.text_steps(cfg.with_(n_block=2, n_steps=1))[0]["q"], "bf16")
    k = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    a = torch.full((2, 32, 128), 5.0, device="cuda")
    l = torch.zeros(2, 32, device="cuda")
    fb.fb_prefix_attn(shape, q, k, k, a, l)
    torch.cuda.synchronize()
    assert torch.all(a == 0) and torch.all(torch.isneginf(l))


def test_prefix_deterministic(fb):
    a1, l1, *_ = run_prefix(fb, W.LONG, 16, 40000)
    a2, l2, *_ = run_prefix(fb, W.LONG, 16, 40000)
    assert np.array_equal(a1, a2) and np.array_equal(l1, l2)
