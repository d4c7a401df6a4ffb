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
