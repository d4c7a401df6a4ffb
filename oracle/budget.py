"""Per-layer update budgets for a stack of layers (SPA-Cache).

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64.

[SPA methodology s2 "adaptive budget allocation"]: the drift of the hidden
states is low in the first layers, peaks in the middle ones and settles in
the last; the update ratio rho(l) of layer l follows a piecewise Gaussian
over depth, so middle layers recompute more tokens and the first and last
ones cache more. The pages give the shape, not its parameters; reading:

* rho(l) = floor + (peak - floor) * g(l), g(l) = exp(-(l - mu)^2 / (2 s^2))
  with s = s_left for l < mu and s = s_right for l >= mu (two half
  Gaussians meeting at the peak layer mu);
* peak is set so that the mean of rho over the L layers equals the target
  mean ratio (the pages' ablation lowers the mean update ratio from 25% to
  16% with the adaptive schedule): peak = floor + (mean - floor) / mean(g);
* the layer's recomputed-token count is n(l) = floor(rho(l) N + 1/2),
  clamped to [0, N].
"""

import math

import numpy as np


def layer_shape(n_layers, mu, s_left, s_right):
    """g(l) for l = 0 .. L-1 (1 at l = mu)."""
    g = np.empty(n_layers)
    for l in range(n_layers):
        s = s_left if l < mu else s_right
        z = (l - mu) / s
        g[l] = math.exp(-0.5 * z * z)
    return g


def layer_ratios(n_layers, mean_ratio, floor, mu, s_left, s_right):
    g = layer_shape(n_layers, mu, s_left, s_right)
    mg = 0.0
    for v in g:
        mg = mg + v
    mg = mg / n_layers
    peak = floor + (mean_ratio - floor) / mg
    return np.array([floor + (peak - floor) * g[l] for l in range(n_layers)])


def layer_counts(n_tok, ratios):
    out = np.empty(len(ratios), dtype=np.int32)
    for l, r in enumerate(ratios):
        n = int(math.floor(r * n_tok + 0.5))
        out[l] = min(max(n, 0), n_tok)
    return out


def layer_taus(ratios, block, base_tau, mean_ratio):
    """Per-layer reuse thresholds of a stack of FlashBlock layers.

    [FB s2 "adaptive reuse strategies"]: a layer reuses its cached pair while
    fewer than tau block tokens changed; [SPA methodology s2]: layers whose
    states drift more get a larger update budget. Reading: a layer's
    staleness tolerance is inversely proportional to its budget, scaled so
    that a layer at the mean budget keeps base_tau:
    tau(l) = floor(base_tau * mean_ratio / ratio(l) + 1/2), clamped to
    [1, block + 1]; a layer with no budget (ratio <= 0) gets block + 1 and so
    never recomputes after the first step of a block.
    """
    out = np.empty(len(ratios), dtype=np.int32)
    never = block + 1
    for l, r in enumerate(ratios):
        if r <= 0:
            out[l] = never
        else:
            t = math.floor(base_tau * mean_ratio / r + 0.5)
            out[l] = min(max(t, 1), never)
    return out


__all__ = ["layer_shape", "layer_ratios", "layer_counts", "layer_taus"]
