"""Benchmark: block-step attention query-tok/s and HBM roofline of the prefix pass.

Workload (one bench step): one block of the long-context text workload,
B = 16 block queries, 32 query / 8 KV heads, head_dim 128, bf16, a static
prefix of 800,000 tokens (token-major [N, Hkv, d] K and V, 3.28 GB), eight
denoising steps driven through fb_step: step 0 computes the block-external
pair, later steps reuse it unless M >= tau = 4 updated tokens (M ~ Binomial(16,
0.3) per step, seeded), and every step recomputes the in-block pass and the
merge. Inputs are resident in HBM before the timed region.

value = query tokens per second = (steps x 8 denoising steps x B) / time.
The roofline entry times the prefix pass alone (fb_prefix_attn: the MFMA
prefix kernel plus its split-K reduce) with HIP events on the stream it is
launched on, and divides the algorithmic bytes (K + V + Q + A_out/L_out) by
that duration; the peak is MI355X's 8 TB/s HBM3E.

cpu_baseline: the fp64 oracle on the host cores for a bounded sample of the
same block (one recompute step and one reuse step, timed), scaled to the
block's mix of recompute and reuse steps.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefix_pass_traffic.json")
KERNEL_SOURCES = ("block_diffusion_attention_amd/csrc/k1_prefix.hip",
                  "block_diffusion_attention_amd/csrc/fb_host.hip")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(n_prefix, block):
    """HBM bytes per prefix pass from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources and this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_source_sha256") != kernel_source_hash()
            or t.get("n_prefix") != n_prefix or t.get("block") != block):
        return None
    return t.get("traffic_bytes_per_pass")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--n-prefix", type=int, default=800000)
    ap.add_argument("--block", type=int, default=16)
    ap.add_argument("--roofline-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the prefix pass over 128k-800k contexts and B in {8, 16}")
    ap.add_argument("--prefix-only", action="store_true",
                    help="profiling mode: run the prefix pass --roofline-reps times, then "
                         "a 1 GiB read + 1 GiB write elementwise kernel (counter "
                         "calibration); prints a short JSON")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FlashBlock step shards by KV head or by "
              "prefix range, which this build does not implement; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_diffusion_attention_amd as fb
    import workloads as W

    fb.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = W.LONG.with_(n_prefix=args.n_prefix, n_block=args.block)
    hq, hkv, d, B, N = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_block, cfg.n_prefix

    t0 = time.time()
    kp, vp = W.prefix_kv(cfg)
    steps = W.text_steps(cfg)
    t_gen = time.time() - t0

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    k_dev, v_dev = bf(kp), bf(vp)
    inputs = [(bf(s["q"]), bf(s["k"]), bf(s["v"]), torch.from_numpy(s["ids"]).to(dev))
              for s in steps]
    shape = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
    stream = torch.cuda.current_stream()

    if args.prefix_only:
        prefix_only(args, fb, shape, inputs[0][0], k_dev, v_dev, B, N, hq, hkv, d, stream)
        return

    step = fb.Step(fb.FB_STEP_TEXT, shape, B, k_dev, v_dev, tau=cfg.tau)
    a_full = torch.empty(B, hq, d, device=dev)
    l_full = torch.empty(B, hq, device=dev)

    def run_block(decisions=None):
        step.new_block()
        for s, (q, k, v, ids) in enumerate(inputs):
            dec = -1 if decisions is None or s == 0 else decisions
            step.step(q, k, v, a_full, l_full, ids=ids, decision=dec)

    # the block's decisions (device-side), read once outside the timed region
    decisions, m_counts = [], []
    step.new_block()
    for s, (q, k, v, ids) in enumerate(inputs):
        step.step(q, k, v, a_full, l_full, ids=ids)
        torch.cuda.synchronize()
        m_counts.append(int(step.m_count.item()))
        decisions.append("init" if s == 0 else ("reuse" if int(step.mask[0].item()) else "recompute"))
    n_compute = sum(1 for x in decisions if x != "reuse")

    for _ in range(args.warmup):
        run_block()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        run_block()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_block = e0.elapsed_time(e1) / args.steps
    n_steps_block = len(inputs)
    value = args.steps * n_steps_block * B / (ms_block * args.steps * 1e-3)

    # ---- roofline: the prefix pass alone, events on its stream -------------
    q0 = inputs[0][0]
    a_out = torch.empty(B, hq, d, device=dev)
    l_out = torch.empty(B, hq, device=dev)
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, B, N), 16), dtype=torch.uint8,
                     device=dev)
    for _ in range(3):
        fb.fb_prefix_attn(shape, q0, k_dev, v_dev, a_out, l_out, ws=ws, stream=stream)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(args.roofline_reps):
        fb.fb_prefix_attn(shape, q0, k_dev, v_dev, a_out, l_out, ws=ws, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    t_prefix = r0.elapsed_time(r1) / args.roofline_reps * 1e-3
    alg_bytes = N * hkv * d * 2 * 2 + B * hq * d * 2 + B * hq * (d + 1) * 4
    achieved = alg_bytes / t_prefix / 1e9

    extra = {}
    # reuse-step floor vs dense recompute step (same block, device-side decisions)
    def time_blocks(dec, reps=10):
        run_block(dec)
        torch.cuda.synchronize()
        x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        x0.record(stream)
        for _ in range(reps):
            run_block(dec)
        x1.record(stream)
        torch.cuda.synchronize()
        return x0.elapsed_time(x1) / reps
    ms_dense_block = time_blocks(0)
    ms_reuse_block = time_blocks(1)
    extra["ms_block_dense_recompute"] = round(ms_dense_block, 4)
    extra["ms_block_forced_reuse"] = round(ms_reuse_block, 4)
    extra["speedup_vs_dense_recompute"] = round(ms_dense_block / ms_block, 3)
    extra["decisions"] = decisions
    extra["m_counts"] = m_counts
    extra["prefix_pass_us"] = round(t_prefix * 1e6, 2)

    if args.sweep:
        sweep = []
        for n_ctx in (131072, 200000, 400000, 800000):
            if n_ctx > N:
                continue
            for b in (8, 16):
                sh = fb.shape_of(hq, hkv, d, cfg.scale, torch.bfloat16)
                qq = inputs[0][0][:b].contiguous()
                kk, vv = k_dev[:n_ctx], v_dev[:n_ctx]
                ao = torch.empty(b, hq, d, device=dev)
                lo = torch.empty(b, hq, device=dev)
                w2 = torch.empty(max(fb.fb_prefix_attn_workspace(sh, b, n_ctx), 16),
                                 dtype=torch.uint8, device=dev)
                for _ in range(3):
                    fb.fb_prefix_attn(sh, qq, kk, vv, ao, lo, ws=w2, stream=stream)
                torch.cuda.synchronize()
                x0, x1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                x0.record(stream)
                for _ in range(20):
                    fb.fb_prefix_attn(sh, qq, kk, vv, ao, lo, ws=w2, stream=stream)
                x1.record(stream)
                torch.cuda.synchronize()
                t = x0.elapsed_time(x1) / 20 * 1e-3
                by = n_ctx * hkv * d * 4 + b * hq * d * 2 + b * hq * (d + 1) * 4
                sweep.append({"n_prefix": n_ctx, "B": b, "prefix_pass_us": round(t * 1e6, 2),
                              "GB_s": round(by / t / 1e9, 1),
                              "frac": round(by / t / 1e9 / PEAK_HBM_GBS, 4)})
        extra["prefix_sweep"] = sweep

    out = {
        "metric": "block-step attention query-tok/s (+ prefix-pass HBM GB/s vs peak)",
        "value": round(value, 2),
        "unit": "query-tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_block, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 prefix K/V and block Q/K/V; token updates "
                "M ~ Binomial(B, 0.3) per denoising step)",
        "config": {"workload": "long-context text block diffusion: 32q/8kv heads, d=128, "
                               "B=%d, prefix %d tokens, 8 denoising steps per block, tau=4; "
                               "one bench step = one block" % (B, N),
                   "n_prefix": N, "block": B, "n_q_heads": hq, "n_kv_heads": hkv,
                   "head_dim": d, "denoising_steps": n_steps_block,
                   "recompute_steps": n_compute},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(N, B),
                     "kernel": "prefix pass (prefix_mfma_kernel + prefix_reduce_kernel)",
                     "alg_bytes_per_launch": alg_bytes},
        "extra": extra,
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, kp, vp, steps, decisions)
    out["extra"]["t_generate_inputs_s"] = round(t_gen, 1)
    print(json.dumps(out), flush=True)


def prefix_only(args, fb, shape, q0, k_dev, v_dev, B, N, hq, hkv, d, stream):
    import torch
    dev = q0.device
    a_out = torch.empty(B, hq, d, device=dev)
    l_out = torch.empty(B, hq, device=dev)
    ws = torch.empty(max(fb.fb_prefix_attn_workspace(shape, B, N), 16), dtype=torch.uint8,
                     device=dev)
    for _ in range(3):
        fb.fb_prefix_attn(shape, q0, k_dev, v_dev, a_out, l_out, ws=ws, stream=stream)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(args.roofline_reps):
        fb.fb_prefix_attn(shape, q0, k_dev, v_dev, a_out, l_out, ws=ws, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    t = r0.elapsed_time(r1) / args.roofline_reps * 1e-3
    # counter calibration: an elementwise kernel that reads exactly 1 GiB and
    # writes exactly 1 GiB (torch.add on uint8; the fill writes 1 GiB)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        torch.add(src, 1, out=dst)
    torch.cuda.synchronize()
    alg = N * hkv * d * 4 + B * hq * d * 2 + B * hq * (d + 1) * 4
    print(json.dumps({"prefix_pass_us": round(t * 1e6, 2), "alg_bytes": alg,
                      "GB_s": round(alg / t / 1e9, 1), "reps": args.roofline_reps,
                      "calibration_copy_bytes": 1 << 30}), flush=True)


def cpu_baseline(cfg, kp, vp, steps, decisions):
    """The fp64 oracle on the host: one recompute step and one reuse step of the
    block, timed, scaled to the block's recompute/reuse mix."""
    import workloads as W
    from oracle.attention import attn_gqa, merge

    kf, vf = W.bf16_to_f32(kp), W.bf16_to_f32(vp)
    st = [dict(q=W.bf16_to_f32(s["q"]), k=W.bf16_to_f32(s["k"]), v=W.bf16_to_f32(s["v"]))
          for s in steps[:2]]
    t0 = time.time()
    ao, lo = attn_gqa(st[0]["q"], kf, vf, cfg.scale)           # recompute: prefix pass
    ai, li = attn_gqa(st[0]["q"], st[0]["k"], st[0]["v"], cfg.scale)
    merge(ao, lo, ai, li)
    t_recompute = time.time() - t0
    t0 = time.time()
    ai, li = attn_gqa(st[1]["q"], st[1]["k"], st[1]["v"], cfg.scale)   # reuse: in-block + merge
    merge(ao, lo, ai, li)
    t_reuse = time.time() - t0
    n_comp = sum(1 for x in decisions if x != "reuse")
    t_block = n_comp * t_recompute + (len(decisions) - n_comp) * t_reuse
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(len(decisions) * cfg.n_block / t_block, 3), "unit": "query-tok/s",
            "cores": cores, "kind": "oracle",
            "sample": "one recompute step (fp64 dense softmax over the %d-token prefix for %d "
                      "queries x 32 heads) and one reuse step, timed; block time = %d x %.2f s + "
                      "%d x %.4f s" % (cfg.n_prefix, cfg.n_block, n_comp, t_recompute,
                                       len(decisions) - n_comp, t_reuse)}


if __name__ == "__main__":
    main()
