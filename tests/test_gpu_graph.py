"""fb_step under HIP graph capture: a whole block's steps recorded once in a
graph (torch.cuda.CUDAGraph over the library's launches) and replayed. The
library issues no memset, copy or synchronisation, so the graph holds only
its kernels. Every replay -- with eager work of the program and
synchronisations between replays -- must reproduce the eager run bit for
bit (same kernels, same inputs, fixed-order reductions), including the
decisions taken on the device."""

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import cpu, dev_tensor

pytestmark = pytest.mark.gpu


def _text_block(fb, cfg, layout):
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, torch.bfloat16)
    kd, vd = dev_tensor(kp, "bf16", layout), dev_tensor(vp, "bf16", layout)
    inputs = [(dev_tensor(s["q"], "bf16"), dev_tensor(s["k"], "bf16"), dev_tensor(s["v"], "bf16"),
               torch.from_numpy(s["ids"]).cuda()) for s in steps]
    return shape, kd, vd, inputs


def _outputs(n, b, hq, d):
    return [(torch.empty(b, hq, d, device="cuda"), torch.empty(b, hq, device="cuda"))
            for _ in range(n)]


def _snapshot(outs, step):
    return [cpu(x) for pair in outs for x in pair] + [cpu(step.a_out), cpu(step.l_out),
                                                      cpu(step.mask), cpu(step.m_count)]


@pytest.mark.parametrize("name,cfg,layout", [
    ("text_32k_b4", W.TEXT, "head"),
    ("long_131k_b16", W.LONG.with_(n_prefix=131072), "head"),
    ("long_60k_b8_token", W.LONG.with_(n_prefix=60000, n_block=8), "tok"),
])
def test_text_block_graph_replays_match_eager(fb, name, cfg, layout):
    shape, kd, vd, inputs = _text_block(fb, cfg, layout)
    hq, d, b = cfg.n_q_heads, cfg.head_dim, cfg.n_block
    step = fb.Step(fb.FB_STEP_TEXT, shape, b, kd, vd, tau=cfg.tau)
    outs = _outputs(len(inputs), b, hq, d)

    def block():
        step.new_block()
        for (q, k, v, ids), (a, l) in zip(inputs, outs):
            step.step(q, k, v, a, l, ids=ids)

    # eager reference (after a warm-up block on a side stream, as capture wants)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        block()
    torch.cuda.current_stream().wait_stream(s)
    block()
    torch.cuda.synchronize()
    want = _snapshot(outs, step)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block()
    # other eager work of the program between replays: a second Step on the
    # same prefix, different outputs
    other = fb.Step(fb.FB_STEP_TEXT, shape, b, kd, vd, tau=cfg.tau)
    oa, ol = torch.empty(b, hq, d, device="cuda"), torch.empty(b, hq, device="cuda")
    for rep in range(4):
        for x in outs:
            x[0].fill_(-3.0)
            x[1].fill_(-3.0)
        step.a_out.fill_(5.0)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(outs, step)
        for i, (x, y) in enumerate(zip(got, want)):
            assert np.array_equal(x, y), (name, rep, i)
        other.new_block()
        for q, k, v, ids in inputs[:3]:
            other.step(q, k, v, oa, ol, ids=ids)
        torch.cuda.synchronize()


def test_sparse_block_graph_replays_match_eager(fb):
    cfg = W.SPARSE.with_(n_prefix=16384, n_steps=6)
    kp, vp = W.prefix_kv(cfg)
    steps = W.sparse_steps(cfg, m_override=[None, 2, 0, 5, 1, 3])
    shape = fb.shape_of(32, 8, 128, cfg.scale, torch.bfloat16)
    kd, vd = dev_tensor(kp, "bf16", "head"), dev_tensor(vp, "bf16", "head")
    inputs = [tuple(dev_tensor(s[n], "bf16") for n in ("q", "k", "v")) for s in steps]
    for reselect in (False, True):
        step = fb.Step(fb.FB_STEP_SPARSE, shape, 8, kd, vd, page_size=cfg.page,
                       k_pages=cfg.k_pages, pct=cfg.pct, reselect=reselect)
        outs = _outputs(len(inputs), 8, 32, 128)

        def block():
            step.new_block()
            for (q, k, v), (a, l) in zip(inputs, outs):
                step.step(q, k, v, a, l)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            block()
        torch.cuda.current_stream().wait_stream(s)
        block()
        torch.cuda.synchronize()
        want = [cpu(x) for pair in outs for x in pair] + [cpu(step.pages), cpu(step.active)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            block()
        for rep in range(3):
            for x in outs:
                x[0].fill_(-3.0)
            step.active.fill_(9)
            g.replay()
            torch.cuda.synchronize()
            got = [cpu(x) for pair in outs for x in pair] + [cpu(step.pages), cpu(step.active)]
            for i, (x, y) in enumerate(zip(got, want)):
                assert np.array_equal(x, y), (reselect, rep, i)
