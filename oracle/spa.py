"""Singular-proxy identification of the tokens to recompute (SPA-Cache).

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 throughout.

[SPA "Proxy singolari", methodology s1 "identification by singular proxies"]:
value-state stability bounds the drift of the attention and FFN outputs, so
the tokens to recompute are found from the value states; to keep that cheap
the value projection W is replaced by its rank-r truncated SVD, the input
states are projected onto that r-dimensional space, each token's proxy is
compared by cosine with the proxy cached for it, and the tokens of lowest
similarity (largest drift) are recomputed. W = U diag(sigma) V^T with V
orthonormal, so the cosine of x U_r diag(sigma_r) equals the cosine of the
rank-r value states x W_r: the stored factor is F = U_r diag(sigma_r) [D, r].

Readings (the pages fix no precision, order or tie rule):

* proxy p = x F, one float64 matrix product (a library primitive; its
  summation order is the library's -- the GPU's proxies are compared with it
  to a rounding tolerance, not bit for bit);
* similarity of token t: the cosine <p_t, c_t> / sqrt(|p_t|^2 |c_t|^2) of
  its proxy and its cached proxy, clamped to [-1, 1]; both norms zero -> 1
  (identical), one zero -> 0. (With the squared norms under one square root,
  a proxy equal to its cache scores exactly 1: sqrt of a rounded square is
  the value itself in binary floating point.)
* the n_select tokens of lowest similarity are recomputed (ties: lower token
  id first); their cached proxies become the current ones; the other tokens
  keep the proxy cached at the step they were last recomputed;
* the first step recomputes every token and caches every proxy.
"""

import math

import numpy as np


def proxy(x, factor):
    """x [N, D], factor [D, r] -> p = x F [N, r] (float64)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(factor, dtype=np.float64)


def proxy_cosine(p, c):
    """Per row, the cosine of proxy p against cached proxy c (conventions above)."""
    p = np.asarray(p, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    sim = np.empty(p.shape[0])
    for t in range(p.shape[0]):
        dot = float(np.dot(p[t], c[t]))
        pp = float(np.dot(p[t], p[t]))
        cc = float(np.dot(c[t], c[t]))
        if pp == 0.0 or cc == 0.0:
            sim[t] = 1.0 if (pp == 0.0 and cc == 0.0) else 0.0
        else:
            sim[t] = min(1.0, max(-1.0, dot / math.sqrt(pp * cc)))
    return sim


def select_lowest(sim, n_select):
    """Token ids of the n_select lowest similarities (ties: lower id), ascending."""
    sim = np.asarray(sim, dtype=np.float64)
    ids = np.arange(sim.size)
    order = np.lexsort((ids, sim))
    return np.sort(order[:int(n_select)]).astype(np.int32)


def spa_run(steps, factor, n_select):
    """The identifier over denoising steps of hidden states x^s [N, D].

    Per step: the proxies; at s = 0 every token is recomputed and cached; at
    s >= 1 the similarities against the cache, the n_select lowest
    recomputed and their cache entries replaced. Records: proxy, sim (None
    at s = 0), selected, mask, cache after the step.
    """
    recs = []
    cache = None
    for s, x in enumerate(steps):
        p = proxy(x, factor)
        n = p.shape[0]
        if s == 0:
            sim, sel = None, np.arange(n, dtype=np.int32)
            cache = p.copy()
        else:
            sim = proxy_cosine(p, cache)
            sel = select_lowest(sim, n_select)
            cache = cache.copy()
            cache[sel] = p[sel]
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        recs.append(dict(step=s, proxy=p, sim=sim, selected=sel, mask=mask, cache=cache))
    return recs


__all__ = ["proxy", "proxy_cosine", "select_lowest", "spa_run"]
