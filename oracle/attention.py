"""Softmax attention with its log-normaliser, and the FlashBlock log-space merge.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain float64 numpy,
no blocking, no fusion, no chunking over the key axis.

Citations are to the pages listed in ``oracle/__init__.py``.
"""

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attn(q, k, v, scale):
    """Softmax attention of query rows over one key/value set.

    [FB s2 "core mechanism"]: a block query attends over a key set J (J_out,
    the tokens outside the block, or J_in, the block's own tokens) and yields
    the output A and the log-normaliser L = log Z, Z the softmax denominator.
    Reading: natural log, Z taken over the *scaled* scores s_j = scale*q.k_j.

    q [R, d], k [N, d], v [N, dv]  ->  A [R, dv], L [R].

    The full R x N score matrix is materialised. Subtracting the row max m is
    only the stable way to evaluate Z: L = m + ln(sum_j exp(s_j - m)).
    An empty key set (N = 0) gives A = 0 and L = -inf, the identity of
    ``merge``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    R, N = q.shape[0], k.shape[0]
    if N == 0:
        return np.zeros((R, v.shape[1])), np.full(R, NEG_INF)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1)
    a = (e @ v) / z[:, None]
    return a, m[:, 0] + np.log(z)


def kv_head_of(h, n_q_heads, n_kv_heads):
    """Grouped-query mapping: query head h reads KV head floor(h * Hkv / Hq).

    The pages do not state the head layout; contiguous groups of Hq/Hkv query
    heads per KV head is the plain reading (equal to h // (Hq/Hkv)).
    """
    return (h * n_kv_heads) // n_q_heads


def attn_gqa(q, k, v, scale, heads=None):
    """Multi-head (grouped-query) attention of block rows over one key set.

    q [n_q, Hq, d]; k, v [N, Hkv, d]. Returns A [n_q, Hq, d], L [n_q, Hq].
    Loops over query heads (optionally only ``heads``); each uses its KV head
    per ``kv_head_of``. Rows of heads not in ``heads`` are left as A = 0,
    L = -inf.
    """
    q = _f64(q)
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    a = np.zeros((n_q, hq, v.shape[2]))
    lse = np.full((n_q, hq), NEG_INF)
    heads = range(hq) if heads is None else heads
    kv_cache = {}
    for h in heads:
        g = kv_head_of(h, hq, hkv)
        if g not in kv_cache:
            kv_cache = {g: (_f64(k[:, g, :]), _f64(v[:, g, :]))}
        kg, vg = kv_cache[g]
        a[:, h, :], lse[:, h] = attn(q[:, h, :], kg, vg, scale)
    return a, lse


def merge(a1, l1, a2, l2):
    """Log-space composition of two partial attentions over disjoint key sets.

    [FB s2 "core mechanism", the A_full equation]: with m = max(L1, L2),
    A = (e^{L1-m} A1 + e^{L2-m} A2) / (e^{L1-m} + e^{L2-m}); the merged
    log-normaliser is L = m + ln(e^{L1-m} + e^{L2-m}) (the log of Z1 + Z2).
    Rows where both sides are empty (m = -inf) give A = 0, L = -inf; a side
    with L = -inf has weight 0, so the other side passes through.

    a* [..., dv], l* [...]; any leading shape.
    """
    a1, l1, a2, l2 = _f64(a1), _f64(l1), _f64(a2), _f64(l2)
    m = np.maximum(l1, l2)
    out_a = np.zeros(np.broadcast_shapes(a1.shape, a2.shape))
    out_l = np.full(m.shape, NEG_INF)
    ok = m > NEG_INF
    w1 = np.exp(l1[ok] - m[ok])
    w2 = np.exp(l2[ok] - m[ok])
    den = w1 + w2
    out_a[ok] = (w1[:, None] * a1[ok] + w2[:, None] * a2[ok]) / den[:, None]
    out_l[ok] = m[ok] + np.log(den)
    return out_a, out_l


def dense_step(q_blk, k_p, v_p, k_blk, v_blk, scale):
    """The dense baseline of one denoising step: attention over prefix and block.

    [FB s1 problem statement]: standard block diffusion recomputes attention
    over the whole KV cache at every step. J = J_out (the prefix) followed by
    J_in (the B block tokens); within the block every query sees every block
    key (bidirectional; the pages state no in-block mask).
    """
    k = np.concatenate([_f64(k_p), _f64(k_blk)], axis=0)
    v = np.concatenate([_f64(v_p), _f64(v_blk)], axis=0)
    return attn_gqa(q_blk, k, v, scale)
