"""Shared helpers for the GPU parity tests (not collected: no test_ prefix).

Tolerances: for bf16 inputs with fp32 accumulation, max |A_gpu - A_oracle|
<= 2e-3 and max |L_gpu - L_oracle| <= 1e-3. Because attention outputs over
long N(0,1) prefixes are small (RMS ~ sqrt(e/N)), the A check also gates the
error relative to the largest reference magnitude (<= 1e-2), so that a
vanishing output cannot pass by being small. fp32 inputs: 1e-5 / 1e-5.
"""

import numpy as np
import torch

import workloads as W

A_TOL_BF16, L_TOL_BF16, REL_TOL = 2e-3, 1e-3, 1e-2
A_TOL_F32, L_TOL_F32 = 1e-5, 1e-5


def dev_tensor(x, dtype, layout="tok", device="cuda"):
    """Workload array [N, H, d] (bf16 bits or float32) -> device tensor view
    [N, H, d]. layout 'head' stores it head-major ([H, N, d] contiguous)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if layout == "head":
        return t.permute(1, 0, 2).contiguous().to(device).permute(1, 0, 2)
    return t.to(device)


def vals(x, dtype):
    return W.values(x, dtype)


def tols(dtype):
    return (A_TOL_BF16, L_TOL_BF16) if dtype == "bf16" else (A_TOL_F32, L_TOL_F32)


def check_a(name, got, ref, atol, rel=REL_TOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % name
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    assert err <= atol, "%s: max|err| %.3g > %.3g (max|ref| %.3g)" % (name, err, atol, scale)
    if scale > 0:
        assert err <= rel * scale, "%s: max|err| %.3g > %g * max|ref| %.3g" % (name, err, rel, scale)
    return err


def check_l(name, got, ref, atol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), "%s: -inf pattern differs" % name
    if (~inf_ref).any():
        err = float(np.max(np.abs(got[~inf_ref] - ref[~inf_ref])))
        assert err <= atol, "%s: max|err| %.3g > %.3g" % (name, err, atol)
        return err
    return 0.0


def cpu(t):
    return t.detach().cpu().numpy()


def run_prefix(fb, cfg, n_q, n_kv, layout="tok", mask=None, q_gain=1.0, seed_variant=0,
               v_edit=None):
    """fb_prefix_attn on seeded inputs of `cfg` (n_q block rows over an n_kv
    prefix) and the oracle's A_out, L_out. Outputs start as 7.0 so rows the
    pass must leave alone can be checked. v_edit(vp) may alter the prefix V
    (stored values) before both sides see it."""
    from oracle.attention import attn_gqa
    cfg = cfg.with_(n_prefix=n_kv, n_block=n_q, q_gain=q_gain)
    kp, vp = W.prefix_kv(cfg, variant=seed_variant)
    if v_edit is not None:
        vp = vp.copy()
        v_edit(vp)
    q = W.text_steps(cfg.with_(n_steps=1), variant=seed_variant)[0]["q"]
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = fb.shape_of(cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.scale, tdt)
    qd = dev_tensor(q, cfg.dtype)
    kd, vd = dev_tensor(kp, cfg.dtype, layout), dev_tensor(vp, cfg.dtype, layout)
    a = torch.full((n_q, cfg.n_q_heads, cfg.head_dim), 7.0, device="cuda")
    l = torch.full((n_q, cfg.n_q_heads), 7.0, device="cuda")
    nbytes = fb.fb_prefix_attn_workspace(shape, n_q, n_kv)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    md = None if mask is None else torch.tensor(mask, dtype=torch.uint8, device="cuda")
    fb.fb_prefix_attn(shape, qd, kd, vd, a, l, mask=md, ws=ws)
    torch.cuda.synchronize()
    ra, rl = attn_gqa(vals(q, cfg.dtype), vals(kp, cfg.dtype), vals(vp, cfg.dtype), cfg.scale)
    return cpu(a), cpu(l), ra, rl, cfg


# ---------------------------------------------------------------- margin guards
#
# Where a float64 value decides an integer result (the active set from the
# query MSE, the recomputed tokens from the proxy similarity), the oracle
# computes the plain definition (an exact mean; a library matrix product and
# the plain cosine) and the GPU its own summation order. The values then
# differ by rounding only, so they are compared to a tolerance, and the
# integer results are compared bit for bit once the oracle's values leave a
# margin around every decision that no rounding difference can cross.

MSE_RTOL = 1e-12        # GPU float64 MSE (its own order) vs the exact mean
MSE_MARGIN = 1e-9       # relative gap the guard requires between distinct MSEs
SIM_ATOL = 1e-10        # GPU proxy cosine vs the oracle's
SIM_MARGIN = 1e-8       # gap the guard requires at the selection boundary


def check_mse(name, got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert np.array_equal(got == 0.0, want == 0.0), "%s: zero pattern differs" % name
    err = np.abs(got - want)
    assert np.all(err <= MSE_RTOL * np.abs(want)), "%s: MSE %s vs %s" % (name, got, want)


def mse_margin_ok(mse):
    """True when the distinct MSE values are more than MSE_MARGIN apart
    (relative), so that any order of the GPU's sums ranks them alike and the
    nearest-rank cutoff picks the same token; equal values (unchanged tokens
    score exactly 0 on both sides) are allowed."""
    u = np.unique(np.asarray(mse, dtype=np.float64))
    if u.size < 2:
        return True
    return bool(np.all(np.diff(u) > MSE_MARGIN * u[1:]))


def sim_margin_ok(sim, n_select):
    """True when the n_select-th lowest and the next similarity are more than
    SIM_MARGIN apart, so the selection cannot flip under rounding."""
    s = np.sort(np.asarray(sim, dtype=np.float64))
    if n_select <= 0 or n_select >= s.size:
        return True
    return bool(s[n_select] - s[n_select - 1] > SIM_MARGIN)
