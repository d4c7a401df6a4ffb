"""QUEST-style page selection and the selected / residual split of the prefix.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[LoSA s2 "optimisation mechanism"]: active tokens run sparse attention with
the QUEST selector; [LoSA s1, s2 "KV union reduction"]: the memory-bound cost
follows the union of the KV positions the queries select, taken over the
active tokens only. [FB s2 "adaptive reuse strategies", sparse
compatibility]: the unselected keys form the cached residual.

The pages name QUEST but do not restate it; the selector used here is the
plain page bound: per page, the elementwise min and max of its keys, and for a
query the upper bound sum_d max(q_d * kmin_d, q_d * kmax_d) of q.k over the
page. Scores are float64 with a sequential sum over d (products of two bf16
values are exact in float64, so the sum's rounding is fixed by its order).
"""

import numpy as np

from .attention import attn, kv_head_of


def n_pages(n_tok, page):
    return (n_tok + page - 1) // page


def page_meta(k, page):
    """Per (KV head, page, dim): min and max of the page's keys.

    k [N, Hkv, d]  ->  kmin, kmax [Hkv, P, d], P = ceil(N / page); the last
    page may hold fewer than ``page`` tokens.
    """
    k = np.asarray(k, dtype=np.float64)
    n, hkv, d = k.shape
    p = n_pages(n, page)
    kmin = np.empty((hkv, p, d))
    kmax = np.empty((hkv, p, d))
    for i in range(p):
        blk = k[i * page:(i + 1) * page]          # [<=page, Hkv, d]
        kmin[:, i, :] = blk.min(axis=0)
        kmax[:, i, :] = blk.max(axis=0)
    return kmin, kmax


def page_bound(q, kmin, kmax):
    """U[t, g, p] = max over the query heads h of group g of
    sum_d max(q[t,h,d] * kmin[g,p,d], q[t,h,d] * kmax[g,p,d]).

    The sum runs sequentially over d = 0 .. d-1 in float64 (vectorised over
    tokens and pages only).
    """
    q = np.asarray(q, dtype=np.float64)
    n_tok, hq, d = q.shape
    hkv, p, _ = kmin.shape
    out = np.full((n_tok, hkv, p), -np.inf)
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        acc = np.zeros((n_tok, p))
        for j in range(d):
            qj = q[:, h, j][:, None]
            lo = qj * kmin[g, :, j][None, :]
            hi = qj * kmax[g, :, j][None, :]
            acc = acc + np.maximum(lo, hi)
        out[:, g, :] = np.maximum(out[:, g, :], acc)
    return out


def page_bound_heads(q, kmin, kmax):
    """The bound before the group maximum: one row per query head.

    U[t, h, p] = sum_d max(q[t,h,d] * kmin[g,p,d], q[t,h,d] * kmax[g,p,d])
    with g the KV head of h, summed sequentially over d in float64 -- the
    selection granularity of one page set per (token, query head).
    """
    q = np.asarray(q, dtype=np.float64)
    n_tok, hq, d = q.shape
    hkv, p, _ = kmin.shape
    out = np.empty((n_tok, hq, p))
    for h in range(hq):
        g = kv_head_of(h, hq, hkv)
        acc = np.zeros((n_tok, p))
        for j in range(d):
            qj = q[:, h, j][:, None]
            acc = acc + np.maximum(qj * kmin[g, :, j][None, :], qj * kmax[g, :, j][None, :])
        out[:, h, :] = acc
    return out


def topk_pages(bound, k):
    """Top-k pages per (token, KV head) under the order (bound desc, page asc).

    bound [B, Hkv, P]  ->  int32 [B, Hkv, k], each row listed in ascending
    page order (the selected set is unique under the tie-break; listing it in
    page order is a canonical form).
    """
    b = np.asarray(bound)
    n_tok, hkv, p = b.shape
    k = int(k)
    out = np.empty((n_tok, hkv, k), dtype=np.int32)
    pages = np.arange(p)
    for t in range(n_tok):
        for g in range(hkv):
            order = np.lexsort((pages, -b[t, g]))   # primary: -bound, then page
            out[t, g] = np.sort(order[:k])
    return out


def token_index(pages, page, n_tok):
    """Token positions covered by a list of pages (clipped to the prefix)."""
    pages = np.asarray(pages, dtype=np.int64)
    idx = (pages[:, None] * page + np.arange(page)[None, :]).ravel()
    return idx[idx < n_tok]


def split_attn(q, k_p, v_p, sel, page, scale, residual=True):
    """Attention of every row over its selected pages, and over the rest.

    q [B, Hq, d]; k_p, v_p [N, Hkv, d]; sel [B, Hkv, k] page ids. Row (t, h)
    uses the selection of its KV head g(h). Returns ((A_sel, L_sel),
    (A_res, L_res)), each A [B, Hq, d] and L [B, Hq]; with
    ``residual=False`` the second pair is None.
    """
    q = np.asarray(q, dtype=np.float64)
    n_tok, hq, d = q.shape
    n, hkv, _ = k_p.shape
    a_sel = np.zeros((n_tok, hq, d))
    l_sel = np.empty((n_tok, hq))
    a_res = np.zeros((n_tok, hq, d)) if residual else None
    l_res = np.empty((n_tok, hq)) if residual else None
    for g in range(hkv):
        kg = np.asarray(k_p[:, g, :], dtype=np.float64)
        vg = np.asarray(v_p[:, g, :], dtype=np.float64)
        heads = [h for h in range(hq) if kv_head_of(h, hq, hkv) == g]
        for t in range(n_tok):
            idx = token_index(sel[t, g], page, n)
            rows = q[t, heads, :]
            a, l_ = attn(rows, kg[idx], vg[idx], scale)
            a_sel[t, heads], l_sel[t, heads] = a, l_
            if residual:
                keep = np.ones(n, dtype=bool)
                keep[idx] = False
                a, l_ = attn(rows, kg[keep], vg[keep], scale)
                a_res[t, heads], l_res[t, heads] = a, l_
    return (a_sel, l_sel), ((a_res, l_res) if residual else None)


def union_size_heads(sel_heads, active, hkv):
    """|union over active tokens t and query heads h of group g of S[t, h]|
    per KV head g, for a selection made per (token, query head).

    sel_heads [B, Hq, k] page ids (the granularity of ``page_bound_heads``).
    """
    sel_heads = np.asarray(sel_heads)
    n_tok, hq, _ = sel_heads.shape
    act = np.nonzero(np.asarray(active))[0]
    out = np.zeros(hkv, dtype=np.int64)
    for g in range(hkv):
        heads = [h for h in range(hq) if kv_head_of(h, hq, hkv) == g]
        if act.size:
            out[g] = np.unique(sel_heads[np.ix_(act, heads)]).size
    return out


def union_size(sel, active):
    """|union over active tokens t of S[t, g]| for every KV head g.

    [LoSA s1]: the memory-bound cost follows the union of selected positions;
    [LoSA s2]: the union is taken over the active tokens only.
    """
    sel = np.asarray(sel)
    act = np.nonzero(np.asarray(active))[0]
    return np.array([np.unique(sel[act, g]).size if act.size else 0
                     for g in range(sel.shape[1])], dtype=np.int64)
