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

* proxy p[t, i] = sum over c of x[t, c] * F[c, i] in float64, taken in fixed
  blocks of ``PROXY_BLOCK`` consecutive c (each block summed in c order, the
  block sums then added in block order). A product of two bf16 (or two fp32)
  values is exact in float64, so each block sum rounds once per term.
* the ranking key of token t is sign(cos) * cos^2 with cos the cosine of its
  proxy and its cached proxy: dot, |p|^2 and |c|^2 summed over i in order
  (multiply, then add), key = dot^2 / (|p|^2 |c|^2), negated when dot < 0 and
  the quotient is not zero; both norms zero -> 1, one zero -> 0. The key is a
  monotone function of the cosine, so the lowest keys are the lowest
  similarities, with no square root.
* the n_select tokens of lowest key are recomputed (ties: lower token id
  first); their cached proxies become the current ones; the other tokens keep
  the proxy cached at the step they were last recomputed.
* the first step recomputes every token and caches every proxy.
"""

import numpy as np

PROXY_BLOCK = 128


def proxy(x, factor):
    """x [N, D], factor [D, r] -> p [N, r] (float64, the blocked order above)."""
    x = np.asarray(x, dtype=np.float64)
    f = np.asarray(factor, dtype=np.float64)
    n, d = x.shape
    total = np.zeros((n, f.shape[1]))
    for b0 in range(0, d, PROXY_BLOCK):
        acc = np.zeros_like(total)
        for c in range(b0, min(d, b0 + PROXY_BLOCK)):
            acc = acc + x[:, c:c + 1] * f[c:c + 1, :]
        total = total + acc
    return total


def proxy_key(p, c):
    """Ranking key sign(cos) cos^2 of proxies p against cached c, per row."""
    p = np.asarray(p, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    n, r = p.shape
    dot = np.zeros(n)
    pp = np.zeros(n)
    cc = np.zeros(n)
    for i in range(r):
        dot = dot + p[:, i] * c[:, i]
        pp = pp + p[:, i] * p[:, i]
        cc = cc + c[:, i] * c[:, i]
    den = pp * cc
    key = np.empty(n)
    for t in range(n):
        if den[t] == 0.0:
            key[t] = 1.0 if (pp[t] == 0.0 and cc[t] == 0.0) else 0.0
        else:
            q = (dot[t] * dot[t]) / den[t]
            key[t] = -q if (dot[t] < 0.0 and q != 0.0) else q
    return key


def select_lowest(key, n_select):
    """Token ids of the n_select lowest keys (ties: lower id), ascending."""
    key = np.asarray(key, dtype=np.float64)
    ids = np.arange(key.size)
    order = np.lexsort((ids, key))
    return np.sort(order[:int(n_select)]).astype(np.int32)


def spa_run(steps, factor, n_select):
    """The identifier over denoising steps of hidden states x^s [N, D].

    Per step: the proxies; at s = 0 every token is recomputed and cached; at
    s >= 1 the keys against the cache, the n_select lowest recomputed and
    their cache entries replaced. Records: proxy, key (None at s = 0),
    selected, mask, cache after the step.
    """
    recs = []
    cache = None
    for s, x in enumerate(steps):
        p = proxy(x, factor)
        n = p.shape[0]
        if s == 0:
            key, sel = None, np.arange(n, dtype=np.int32)
            cache = p.copy()
        else:
            key = proxy_key(p, cache)
            sel = select_lowest(key, n_select)
            cache = cache.copy()
            cache[sel] = p[sel]
        mask = np.zeros(n, dtype=bool)
        mask[sel] = True
        recs.append(dict(step=s, proxy=p, key=key, selected=sel, mask=mask, cache=cache))
    return recs


__all__ = ["PROXY_BLOCK", "proxy", "proxy_key", "select_lowest", "spa_run"]
