"""Plain, slow fp64 CPU oracle for the FlashBlock block-diffusion attention step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
anything in this package: only the test suite, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (no kernels, headers, helpers or tables); both sides only receive the
same seeded inputs from ``workloads``.

Pages cited (by title, section and equation; the pages are machine summaries
of the papers):

* [FB]   "FlashBlock: Attention Caching for Efficient Long-Context Block
  Diffusion", technical summary (gist.science/{it,ko,de}/paper/2602.05305):
  s1 problem statement; s2 method -- "core mechanism" (the split into A_in
  over J_in and A_out over J_out, the cached pair (A_out, L_out = log Z_out)
  and the log-space composition equation for A_full), "adaptive reuse
  strategies" (threshold tau on the updated-token count M, per-head
  similarity against gamma, sparse-attention compatibility).
* [SPA]  "Proxy singolari per la caching adattiva nei modelli linguistici
  diffusivi" (SPA-Cache), technical summary (gist.science/it/paper/2602.02544):
  methodology s1 identification by singular proxies (truncated SVD of the
  value projection, cosine against the cached proxy, lowest similarity
  recomputed), s2 adaptive budget allocation (per-layer update ratio, a
  piecewise Gaussian over depth).
* [LoSA] "LoSA: Locality Aware Sparse Attention for Block-Wise Diffusion
  Language Models" (gist.science/it/paper/2604.12056): s1 KV inflation;
  s2 methodology -- token classification by query MSE, reuse for stable
  tokens, QUEST-selected sparse attention for active tokens, union over the
  active set only, dense first step.

Modules:

* ``attention``  -- softmax attention with its log-normaliser, GQA, the
  log-space merge, the dense per-step reference.
* ``controller`` -- updated-token count, per-head cosine similarity, active-set
  MSE and percentile cutoff, and the per-step FlashBlock paths (text, video,
  sparse) that use them.
* ``quest``      -- page min/max metadata, the QUEST-style page bound, top-k
  page selection, and the selected/residual split of the prefix.
* ``growing``    -- the outer loop over blocks: each finished block's keys
  and values join the prefix cache before the next block.
* ``spa``        -- the singular-proxy identifier: rank-r proxies of the value
  states, their cosine against the cached proxies, the least similar tokens.
* ``budget``     -- per-layer update budgets over depth (piecewise Gaussian).

All arithmetic is float64 on the exact upcast of the bf16 (or fp32) input
bits. Every function is pinned by the ``-m "not gpu"`` tests against closed
forms, invariants, library routines or brute force on tiny inputs; none is
"parity unpinned".
"""

from . import attention, budget, controller, growing, quest, spa  # noqa: F401
