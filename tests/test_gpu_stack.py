"""A stack of FlashBlock text layers under per-layer reuse budgets: every
layer has its own prefix K/V and block Q/K/V, all layers see the same token
updates, and each layer's fb_step runs with the reuse threshold the depth
schedule assigns it (fb_layer_budgets -> fb_layer_taus). Every layer's
decisions, counts, cached pair and merged output against the oracle's text
controller with that layer's threshold, every step."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import budget as OB
from oracle import controller as OC
from _helpers import check_a, check_l, cpu, dev_tensor, vals

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_layers,n_prefix,block,layout", [(4, 6000, 16, "head"),
                                                            (6, 3000, 8, "tok")])
def test_layer_stack_with_depth_thresholds(fb, n_layers, n_prefix, block, layout):
    cfg = W.LONG.with_(n_prefix=n_prefix, n_block=block, n_steps=8)
    mu = (n_layers - 1) / 2.0
    ratios, _ = fb.fb_layer_budgets(n_layers, block, 0.16, 0.04, mu, n_layers / 5.0,
                                    n_layers / 8.0)
    taus = fb.fb_layer_taus(block, cfg.tau, 0.16, ratios)
    want = OB.layer_taus(OB.layer_ratios(n_layers, 0.16, 0.04, mu, n_layers / 5.0,
                                         n_layers / 8.0), block, cfg.tau, 0.16)
    assert taus == want.tolist()
    assert len(set(taus)) > 1
    layers = W.stack_layers(cfg, n_layers)
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, torch.bfloat16)
    steps_dev, got = [], []
    for l, (kp, vp, steps) in enumerate(layers):
        st = fb.Step(fb.FB_STEP_TEXT, shape, block, dev_tensor(kp, "bf16", layout),
                     dev_tensor(vp, "bf16", layout), tau=taus[l])
        steps_dev.append(st)
        got.append([])
    # a model's order: every layer at step s, then step s + 1
    for s in range(cfg.n_steps):
        for l, (kp, vp, steps) in enumerate(layers):
            st, x = steps_dev[l], steps[s]
            a = torch.empty(block, cfg.n_q_heads, cfg.head_dim, device="cuda")
            lf = torch.empty(block, cfg.n_q_heads, device="cuda")
            st.step(dev_tensor(x["q"], "bf16"), dev_tensor(x["k"], "bf16"),
                    dev_tensor(x["v"], "bf16"), a, lf, ids=torch.from_numpy(x["ids"]).cuda())
            torch.cuda.synchronize()
            got[l].append((cpu(a), cpu(lf), int(st.m_count.item()), cpu(st.mask), cpu(st.a_out),
                           cpu(st.l_out)))
    decisions = []
    for l, (kp, vp, steps) in enumerate(layers):
        ks = [dict(q=vals(x["q"], "bf16"), k=vals(x["k"], "bf16"), v=vals(x["v"], "bf16"),
                   ids=x["ids"]) for x in steps]
        recs = OC.text_block(ks, vals(kp, "bf16"), vals(vp, "bf16"), cfg.scale, taus[l],
                             with_dense=False)
        decisions.append([r["decision"] for r in recs])
        for s, (rec, (a, lf, mc, mask, a_out, l_out)) in enumerate(zip(recs, got[l])):
            tag = "layer %d (tau %d) step %d" % (l, taus[l], s)
            if s > 0:
                assert mc == rec["m_count"], tag
            assert np.all(mask == (1 if rec["decision"] == OC.REUSE else 0)), tag
            check_a(tag + " A_out", a_out, rec["a_out"], 2e-3)
            check_l(tag + " L_out", l_out, rec["l_out"], 1e-3)
            check_a(tag + " A_full", a, rec["a_full"], 2e-3)
            check_l(tag + " L_full", lf, rec["l_full"], 1e-3)
    # the same token updates, different thresholds: some step where one
    # layer reuses and another recomputes
    assert any(len({d[s] for d in decisions}) > 1 for s in range(1, cfg.n_steps))
