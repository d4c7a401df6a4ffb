"""The outer loop over blocks: the prefix grows by each finished block.

TEST INFRASTRUCTURE ONLY (see the package docstring). Float64 throughout.

[FB s1 problem statement]: block diffusion decodes block after block with a
KV cache; every denoising step of a block attends over the whole cache, and
the cache grows as blocks finish. [FB s2 "core mechanism"]: within a block,
the tokens outside it (J_out) are that cache. Reading used here: when a
block's last denoising step is done, its keys and values at that step join
the cache after the tokens already in it, in block order; the next block
starts with no cached pair (its first step computes over the grown cache).
"""

import numpy as np


def append_block(k_p, v_p, k_blk, v_blk):
    """The grown cache: the block's B tokens follow the prefix's N tokens.

    k_p, v_p [N, Hkv, d]; k_blk, v_blk [B, Hkv, d]  ->  [N + B, Hkv, d].
    """
    k = np.concatenate([np.asarray(k_p), np.asarray(k_blk)], axis=0)
    v = np.concatenate([np.asarray(v_p), np.asarray(v_blk)], axis=0)
    return k, v


def run_blocks(blocks, k_p, v_p, block_fn, **kw):
    """Denoise blocks one after another over a growing cache.

    ``blocks`` is a list of per-block step lists (each as ``block_fn``
    takes them: dicts with q, k, v and, for text, ids). For block b,
    ``block_fn(steps, k_cache, v_cache, **kw)`` runs over the cache holding
    the initial prefix and the finished blocks 0 .. b-1; then the block's
    last step's k, v are appended.

    Returns (per-block list of dict(n_prefix, recs), (k_cache, v_cache) after
    the last block).
    """
    out = []
    for steps in blocks:
        recs = block_fn(steps, k_p, v_p, **kw)
        out.append(dict(n_prefix=int(np.asarray(k_p).shape[0]), recs=recs))
        k_p, v_p = append_block(k_p, v_p, steps[-1]["k"], steps[-1]["v"])
    return out, (k_p, v_p)


__all__ = ["append_block", "run_blocks"]
