"""Reuse controllers and the per-step FlashBlock paths (text, video, sparse).

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 throughout;
the active-set MSE is the exact mean of the squared query changes, taken in
rational arithmetic and rounded once, so no order of operations enters it.

Citations are to the pages listed in ``oracle/__init__.py``.
"""

import math
from fractions import Fraction

import numpy as np

from .attention import attn_gqa, dense_step, merge, NEG_INF
from . import quest

INIT, REUSE, RECOMPUTE = "init", "reuse", "recompute"


# --------------------------------------------------------------------------
# decisions
# --------------------------------------------------------------------------

def count_updated(ids_prev, ids_cur):
    """M: how many block positions hold a different token id than one step ago.

    [FB s2 "adaptive reuse strategies", threshold reuse]: the controller
    counts the tokens updated at step s+1. Reading: the per-step count of
    positions whose id changed since the previous step.
    """
    a = np.asarray(ids_prev)
    b = np.asarray(ids_cur)
    return int(np.count_nonzero(a != b))


def text_reuse(m_count, tau):
    """Reuse the cached pair iff M < tau (strict); recompute iff M >= tau.

    [FB s2 "adaptive reuse strategies", threshold reuse].
    """
    return m_count < tau


def head_cosine(a_cur, a_prev):
    """Per-head similarity of two block-external outputs.

    [FB s2 "adaptive reuse strategies", per-head selection]: the method
    estimates one similarity per attention head. Reading: the cosine of the
    head's output flattened over all block queries and dims,
    <A_c, A_p> / (|A_c| |A_p|), in float64, clamped to [-1, 1] (the range of
    a cosine; rounding can step just outside it). A zero-norm side gives 1
    when both sides are all-zero (identical outputs), else 0.

    a_cur, a_prev [n_q, H, d]  ->  sim [H] float64.
    """
    a = np.asarray(a_cur, dtype=np.float64)
    b = np.asarray(a_prev, dtype=np.float64)
    hq = a.shape[1]
    sim = np.empty(hq)
    for h in range(hq):
        x = a[:, h, :].ravel()
        y = b[:, h, :].ravel()
        dot = float(np.dot(x, y))
        nx = math.sqrt(float(np.dot(x, x)))
        ny = math.sqrt(float(np.dot(y, y)))
        if nx * ny == 0.0:
            sim[h] = 1.0 if (nx == 0.0 and ny == 0.0) else 0.0
        else:
            sim[h] = min(1.0, max(-1.0, dot / (nx * ny)))
    return sim


def head_reuse(sim, gamma):
    """A head reuses its cached output iff its similarity is strictly above gamma.

    [FB s2 "adaptive reuse strategies", per-head selection].
    """
    return np.asarray(sim) > gamma


def active_mse(q_prev, q_cur):
    """Locality score per block token: mean squared change of its query.

    [LoSA s2 "token classification", "workflow"]: the score is the MSE
    between a token's query at step t and at step t-1, over all query heads
    and dims. The pages fix no precision or order; reading: the exact mean of
    the squared differences of the float64 inputs (every difference, square
    and the sum taken in rational arithmetic), rounded once to float64. The
    result depends on no summation order.

    q_prev, q_cur [B, Hq, d]  ->  mse [B] float64.
    """
    a = np.asarray(q_prev, dtype=np.float64)
    b = np.asarray(q_cur, dtype=np.float64)
    n_tok = a.shape[0]
    a = a.reshape(n_tok, -1)
    b = b.reshape(n_tok, -1)
    n = a.shape[1]
    out = np.empty(n_tok)
    for t in range(n_tok):
        total = sum((Fraction(y) - Fraction(x)) ** 2 for x, y in zip(a[t].tolist(), b[t].tolist()))
        out[t] = float(total / n)          # one correctly rounded division
    return out


def percentile_cutoff(mse, pct=25):
    """Nearest-rank percentile: the ceil(pct * B / 100)-th smallest value
    (the ceiling taken exactly, in integers).

    Reading of the 25th-percentile cutoff in the sparse workload: nearest
    rank (for B = 8 and pct = 25 it is the 2nd smallest).
    """
    x = np.sort(np.asarray(mse, dtype=np.float64))
    rank = max(1, -(-int(pct) * len(x) // 100))   # exact integer ceil
    return float(x[rank - 1])


def active_set(mse, pct=25):
    """Active tokens: MSE strictly above the percentile cutoff [LoSA s2]."""
    mse = np.asarray(mse, dtype=np.float64)
    return mse > percentile_cutoff(mse, pct)


# --------------------------------------------------------------------------
# text: threshold reuse of the block-external pair
# --------------------------------------------------------------------------

def text_block(steps, k_p, v_p, scale, tau, with_dense=True, force=None,
               since_refresh=False):
    """FlashBlock over one block of denoising steps with the count controller.

    ``steps`` is a list of dicts with q, k, v [B, H*, d] and ids [B] for each
    denoising step. Per step s ([FB s2 "core mechanism" and threshold reuse]):

    * s = 0: no cached pair exists, so (A_out, L_out) is computed over the
      prefix and cached (decision "init"; the dense first step of a block).
    * s >= 1: M = count_updated(ids^{s-1}, ids^s). If M < tau the cached pair
      is reused; otherwise it is recomputed with the current queries and the
      cache is overwritten. The reused pair is the one from the most recent
      compute step.
    * every step: (A_in, L_in) over the B block keys with the current block
      Q/K/V, and A_full = merge(A_out, L_out, A_in, L_in).

    ``force`` (optional list of decisions per step) overrides the controller
    for s >= 1 ("reuse" / "recompute"), for the forced-reuse curves.

    ``since_refresh``: the variant reading of M that counts the positions
    whose id differs from the id they held at the last compute step (the
    drift of the cached pair) instead of one step ago. With a recompute at
    every step the two readings coincide.

    Returns one record per step: decision, M, the cached pair in use, the
    in-block pair, the merged pair, the per-row stale flag (the row's id
    differs from the id it had at the last compute step), and, with
    ``with_dense``, the dense reference (the method's approximation is the
    gap to it on stale rows; it is not a parity target).
    """
    recs = []
    a_out = l_out = None
    ids_at_refresh = None
    for s, st in enumerate(steps):
        if s == 0:
            m_count, decision = None, INIT
        else:
            ref = ids_at_refresh if since_refresh else steps[s - 1]["ids"]
            m_count = count_updated(ref, st["ids"])
            if force is not None and force[s] is not None:
                decision = force[s]
            else:
                decision = REUSE if text_reuse(m_count, tau) else RECOMPUTE
        if decision != REUSE:
            a_out, l_out = attn_gqa(st["q"], k_p, v_p, scale)
            ids_at_refresh = np.array(st["ids"], copy=True)
        a_in, l_in = attn_gqa(st["q"], st["k"], st["v"], scale)
        a_full, l_full = merge(a_out, l_out, a_in, l_in)
        rec = dict(step=s, decision=decision, m_count=m_count,
                   a_out=a_out, l_out=l_out, a_in=a_in, l_in=l_in,
                   a_full=a_full, l_full=l_full,
                   stale=np.asarray(st["ids"]) != ids_at_refresh)
        if with_dense:
            rec["a_dense"], rec["l_dense"] = dense_step(
                st["q"], k_p, v_p, st["k"], st["v"], scale)
        recs.append(rec)
    return recs


# --------------------------------------------------------------------------
# video: per-head reuse with a similarity probe
# --------------------------------------------------------------------------

def video_block(steps, k_p, v_p, scale, gamma, with_dense=False):
    """FlashBlock over one block with per-head reuse decided by similarity.

    [FB s2 "adaptive reuse strategies", per-head selection]: only heads whose
    similarity is above gamma reuse the cache. The pages do not say when the
    similarity is measured; the reading used (a probe protocol):

    * s = 0: every head computes (A_out, L_out); cached ("init").
    * s = 1: every head computes a fresh probe; sim_h = cos(cache_h, probe_h);
      the cache takes the probe; the next step's flag is sim_h > gamma.
    * s >= 2: heads flagged 1 reuse their cache. Heads flagged 0 recompute,
      refresh sim_h = cos(previous cache_h, fresh_h), take the fresh output
      into the cache, and set their flag for the next step to sim_h > gamma.
    * every step: fresh in-block pair and A_full = merge for every head.

    Returns per-step records with the per-head reuse flags used at that step,
    the similarity after the step, and the outputs.
    """
    recs = []
    hq = steps[0]["q"].shape[1]
    reuse = np.zeros(hq, dtype=bool)
    sim = np.full(hq, np.nan)
    a_out = l_out = None
    for s, st in enumerate(steps):
        used = reuse.copy()
        if s == 0:
            a_out, l_out = attn_gqa(st["q"], k_p, v_p, scale)
            decisions = [INIT] * hq
        else:
            heads = [h for h in range(hq) if not used[h]]
            fresh_a, fresh_l = attn_gqa(st["q"], k_p, v_p, scale, heads=heads)
            new_sim = head_cosine(fresh_a, a_out)
            a_out = a_out.copy()
            l_out = l_out.copy()
            for h in heads:
                sim[h] = new_sim[h]
                a_out[:, h, :] = fresh_a[:, h, :]
                l_out[:, h] = fresh_l[:, h]
                reuse[h] = head_reuse(sim[h], gamma)
            decisions = [REUSE if used[h] else RECOMPUTE for h in range(hq)]
        a_in, l_in = attn_gqa(st["q"], st["k"], st["v"], scale)
        a_full, l_full = merge(a_out, l_out, a_in, l_in)
        rec = dict(step=s, decisions=decisions, reuse_used=used,
                   sim=sim.copy(), reuse_next=reuse.copy(),
                   a_out=a_out, l_out=l_out, a_in=a_in, l_in=l_in,
                   a_full=a_full, l_full=l_full)
        if with_dense:
            rec["a_dense"], rec["l_dense"] = dense_step(
                st["q"], k_p, v_p, st["k"], st["v"], scale)
        recs.append(rec)
    return recs


# --------------------------------------------------------------------------
# sparse: QUEST-selected pages, cached residual, LoSA active set
# --------------------------------------------------------------------------

def sparse_block(steps, k_p, v_p, scale, k_pages, page=16, pct=25,
                 with_dense=False):
    """FlashBlock's residual reuse over a sparse (page-selected) prefix.

    [FB s2 "adaptive reuse strategies", sparse compatibility]: the keys a
    sparse attention leaves out form the block-external set, and their
    residual contribution is cached and merged. [LoSA s2]: stable tokens
    reuse the previous prefix result; active tokens (query MSE above a cutoff)
    run sparse attention over QUEST-selected KV; the first step is dense.

    Reading used:

    * s = 0 (refresh): page metadata and the bound U from the current
      queries; top-``k_pages`` pages per (token, KV head). Per row the prefix
      splits into the selected pages (A_sel, L_sel) and the rest
      (A_res, L_res); A_out = merge of the two (the dense prefix result).
      Every token is active.
    * s >= 1: active tokens (``active_set`` of the query MSE against the
      previous step) recompute A_sel over their fixed page set with the
      current query and merge it with the cached residual; stable tokens keep
      their last A_out.
    * every step: fresh in-block pair, A_full = merge.

    Returns records with the selection, the active set, the per-KV-head union
    size of selected pages over the active tokens, and the outputs.
    """
    recs = []
    kmin, kmax = quest.page_meta(k_p, page)
    sel = None
    a_res = l_res = a_out = l_out = None
    n_tok, hq = steps[0]["q"].shape[:2]
    for s, st in enumerate(steps):
        if s == 0:
            bound = quest.page_bound(st["q"], kmin, kmax)
            sel = quest.topk_pages(bound, k_pages)
            (a_sel, l_sel), (a_res, l_res) = quest.split_attn(
                st["q"], k_p, v_p, sel, page, scale)
            a_out, l_out = merge(a_sel, l_sel, a_res, l_res)
            active = np.ones(n_tok, dtype=bool)
            mse = None
        else:
            mse = active_mse(steps[s - 1]["q"], st["q"])
            active = active_set(mse, pct)
            a_out = a_out.copy()
            l_out = l_out.copy()
            rows = np.nonzero(active)[0]
            if rows.size:
                (a_sel, l_sel), _ = quest.split_attn(
                    st["q"][rows], k_p, v_p, sel[rows], page, scale,
                    residual=False)
                a_new, l_new = merge(a_sel, l_sel, a_res[rows], l_res[rows])
                a_out[rows] = a_new
                l_out[rows] = l_new
        a_in, l_in = attn_gqa(st["q"], st["k"], st["v"], scale)
        a_full, l_full = merge(a_out, l_out, a_in, l_in)
        rec = dict(step=s, active=active, mse=mse, sel=sel,
                   union=quest.union_size(sel, active),
                   a_res=a_res, l_res=l_res, a_out=a_out, l_out=l_out,
                   a_in=a_in, l_in=l_in, a_full=a_full, l_full=l_full)
        if with_dense:
            rec["a_dense"], rec["l_dense"] = dense_step(
                st["q"], k_p, v_p, st["k"], st["v"], scale)
        recs.append(rec)
    return recs


# --------------------------------------------------------------------------
# LoSA per step: re-selected pages for active tokens, no residual
# --------------------------------------------------------------------------

def losa_block(steps, k_p, v_p, scale, k_pages, page=16, pct=25, with_dense=False):
    """LoSA's own step: sparse attention for active tokens, reuse for stable ones.

    [LoSA s2 "token classification", "optimisation mechanism", "workflow"]:

    * s = 0: dense attention over the prefix for every token (the dense
      initialisation); every token is active.
    * s >= 1: active tokens (``active_set`` of the query MSE against the
      previous step) attend only to the pages the QUEST-style selector picks
      with their current query -- the selection is made again at every step
      and nothing stands in for the pages left out (no cached residual);
      stable tokens reuse the prefix result of the previous step.
    * every step: fresh in-block pair, A_full = merge.

    The selection granularity is one page set per (token, KV head), bound
    maximised over the group's query heads (as in ``sparse_block``). It is
    made for every token (stable ones included) so that the KV inflation of
    selecting for the whole block can be set against the active-only union
    [LoSA s1, s2 "KV union reduction"].

    Records: active, mse, sel [B, Hkv, k], union (active tokens), union_all
    (all B tokens), and the outputs.
    """
    recs = []
    kmin, kmax = quest.page_meta(k_p, page)
    a_out = l_out = None
    n_tok = steps[0]["q"].shape[0]
    for s, st in enumerate(steps):
        bound = quest.page_bound(st["q"], kmin, kmax)
        sel = quest.topk_pages(bound, k_pages)
        if s == 0:
            a_out, l_out = attn_gqa(st["q"], k_p, v_p, scale)
            active = np.ones(n_tok, dtype=bool)
            mse = None
        else:
            mse = active_mse(steps[s - 1]["q"], st["q"])
            active = active_set(mse, pct)
            a_out = a_out.copy()
            l_out = l_out.copy()
            rows = np.nonzero(active)[0]
            if rows.size:
                (a_sel, l_sel), _ = quest.split_attn(
                    st["q"][rows], k_p, v_p, sel[rows], page, scale, residual=False)
                a_out[rows] = a_sel
                l_out[rows] = l_sel
        a_in, l_in = attn_gqa(st["q"], st["k"], st["v"], scale)
        a_full, l_full = merge(a_out, l_out, a_in, l_in)
        rec = dict(step=s, active=active, mse=mse, sel=sel,
                   union=quest.union_size(sel, active),
                   union_all=quest.union_size(sel, np.ones(n_tok, dtype=bool)),
                   a_out=a_out, l_out=l_out, a_in=a_in, l_in=l_in,
                   a_full=a_full, l_full=l_full)
        if with_dense:
            rec["a_dense"], rec["l_dense"] = dense_step(
                st["q"], k_p, v_p, st["k"], st["v"], scale)
        recs.append(rec)
    return recs


__all__ = [
    "INIT", "REUSE", "RECOMPUTE", "count_updated", "text_reuse",
    "head_cosine", "head_reuse", "active_mse", "percentile_cutoff",
    "active_set", "text_block", "video_block", "sparse_block", "losa_block",
    "NEG_INF",
]
