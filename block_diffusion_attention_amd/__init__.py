"""MI355X (gfx950) FlashBlock block-diffusion attention step.

The compute lives in ``libflashblock.so`` (hand-written HIP kernels behind a
C ABI, ``include/flashblock.h``); this package is a thin ctypes binding with
the same entry-point names plus ``Step``, a helper that allocates the device
buffers one block's ``fb_step`` calls use. PyTorch supplies device memory and
streams only.
"""

import torch

from . import _abi
from ._abi import (  # noqa: F401
    ABI_VERSION, FB_BF16, FB_F32, FB_OK, FB_ERR_DEVICE, FB_ERR_INVALID_ARGUMENT,
    FB_ERR_UNSUPPORTED, FB_ERR_WORKSPACE_TOO_SMALL, FB_REUSE_ACTIVE_MSE, FB_REUSE_COUNT,
    FB_REUSE_HEAD_COS, FB_SEL_DENSE, FB_SEL_GATHER, FB_SEL_SPLIT, FB_STEP_SPARSE,
    FB_STEP_TEXT, FB_STEP_VIDEO, LIB_PATH, SYMBOLS, FlashBlockError, dtype_code,
    fb_abi_version, fb_attn_shape, fb_block_attn_merge, fb_block_attn_merge_workspace,
    fb_kv_append, fb_kv_cache, fb_layer_budgets, fb_layer_taus, fb_proxy_args, fb_proxy_decide, fb_proxy_decide_workspace,
    proxy_args, fb_page_bitmap, fb_page_meta, fb_page_meta_update, fb_page_sel, fb_page_select,
    fb_page_select_workspace, fb_prefix_attn, fb_prefix_attn_noalloc, fb_prefix_attn_workspace,
    fb_reuse_args, NOALLOC_SCRATCH_BYTES,
    fb_reuse_decide, fb_reuse_decide_workspace, fb_status_string, fb_step, fb_step_args,
    fb_step_next_block, fb_step_state, fb_step_workspace, fb_tensor, load, page_sel, ptr,
    shape_of, stream_of, tensor_of, tensors_of)


class KVCache:
    """Device storage for a prefix KV cache that grows by whole blocks.

    capacity tokens of K and V, [capacity, Hkv, d] viewed; ``layout`` "head"
    stores each KV head's tokens contiguously (Hkv x capacity x d), "token"
    stores tokens contiguously (capacity x Hkv x d). ``k_prefix`` and
    ``v_prefix`` view the n_tok tokens in use; ``append`` adds a finished
    block (fb_kv_append).
    """

    def __init__(self, capacity, n_kv_heads, head_dim, dtype, device, layout="head"):
        load()
        if layout == "head":
            self._k = torch.empty(n_kv_heads, capacity, head_dim, device=device, dtype=dtype)
            self._v = torch.empty_like(self._k)
            self.k_all, self.v_all = self._k.permute(1, 0, 2), self._v.permute(1, 0, 2)
        elif layout == "token":
            self._k = torch.empty(capacity, n_kv_heads, head_dim, device=device, dtype=dtype)
            self._v = torch.empty_like(self._k)
            self.k_all, self.v_all = self._k, self._v
        else:
            raise ValueError("layout must be 'head' or 'token'")
        self.cache = fb_kv_cache(self._k.data_ptr(), self._v.data_ptr(), int(capacity), 0,
                                 self.k_all.stride(0), self.k_all.stride(1))

    @property
    def n_tok(self):
        return int(self.cache.n_tok)

    @property
    def capacity(self):
        return int(self.cache.capacity)

    @property
    def k_prefix(self):
        return self.k_all[:self.n_tok]

    @property
    def v_prefix(self):
        return self.v_all[:self.n_tok]

    def append(self, shape, k_blk, v_blk, stream=None):
        fb_kv_append(shape, self.cache, k_blk, v_blk, stream)


class Step:
    """One block's fb_step state and the caller-owned device buffers behind it.

    mode: FB_STEP_TEXT / FB_STEP_VIDEO / FB_STEP_SPARSE. k_prefix, v_prefix:
    [n_kv, Hkv, d] tensors (any token/head strides), or ``cache`` (a
    KVCache): the prefix is then the cache's tokens in use, ``next_block``
    appends a finished block to it and starts the next block, and SPARSE
    page metadata is kept for the cache's capacity and updated
    incrementally. ``new_block()`` restarts the step counter over the same
    prefix (the next call recomputes the cached pair). ``since_refresh``:
    TEXT counts the ids changed since the last recompute step. ``reselect``:
    SPARSE runs LoSA's own step (dense first step, pages chosen again at
    every step, no residual). ``sel_bitmap``: SPARSE keeps a selection as
    bitmaps in a buffer of its own: in residual mode the refresh step's, so
    later steps run no selection prep; with ``reselect`` each step's top-k
    writes its fresh selection there (False: a selection prep every step).
    """

    def __init__(self, mode, shape, n_q, k_prefix=None, v_prefix=None, tau=0, gamma=0.0,
                 page_size=16, k_pages=0, pct=25, device=None, cache=None,
                 since_refresh=False, reselect=False, sel_bitmap=True):
        load()
        self.cache = cache
        if cache is not None:
            k_prefix, v_prefix = cache.k_prefix, cache.v_prefix
        dev = device or k_prefix.device
        hq, d = shape.n_q_heads, shape.head_dim
        f32 = dict(device=dev, dtype=torch.float32)
        self.shape = shape
        self.n_q = n_q
        self.k_prefix, self.v_prefix = k_prefix, v_prefix
        self.a_out = torch.zeros(n_q, hq, d, **f32)
        self.l_out = torch.zeros(n_q, hq, **f32)
        self._masks = [torch.zeros(hq, device=dev, dtype=torch.uint8),
                       torch.zeros(hq, device=dev, dtype=torch.uint8)]
        self.m_count = torch.zeros(1, device=dev, dtype=torch.int32)
        self.ids_prev = torch.zeros(n_q, device=dev, dtype=torch.int32)
        st = fb_step_state()
        st.shape = shape
        st.mode = int(mode)
        st.n_q = int(n_q)
        if cache is not None:      # the cache's storage, also while it is empty
            c = cache.cache
            st.k_prefix = fb_tensor(c.k, c.n_tok, c.stride_tok, c.stride_head)
            st.v_prefix = fb_tensor(c.v, c.n_tok, c.stride_tok, c.stride_head)
        else:
            _, st.k_prefix, st.v_prefix = tensors_of(shape, None, k_prefix, v_prefix)
        st.tau = int(tau)
        st.gamma = float(gamma)
        st.page_size = int(page_size)
        st.k_pages = int(k_pages)
        st.pct = int(pct)
        st.a_out, st.l_out = ptr(self.a_out), ptr(self.l_out)
        st.mask, st.mask_next = ptr(self._masks[0]), ptr(self._masks[1])
        st.m_count, st.ids_prev = ptr(self.m_count), ptr(self.ids_prev)
        if mode == FB_STEP_VIDEO:
            self.a_probe = torch.zeros(n_q, hq, d, **f32)
            self.l_probe = torch.zeros(n_q, hq, **f32)
            self.sim = torch.full((hq,), float("nan"), device=dev, dtype=torch.float64)
            st.a_probe, st.l_probe, st.sim = ptr(self.a_probe), ptr(self.l_probe), ptr(self.sim)
        if mode == FB_STEP_SPARSE:
            hkv = shape.n_kv_heads
            n_tok = cache.capacity if cache is not None else k_prefix.shape[0]
            n_pages = (n_tok + page_size - 1) // page_size
            kdt = k_prefix.dtype
            self.a_res = torch.zeros(n_q, hq, d, **f32)
            self.l_res = torch.zeros(n_q, hq, **f32)
            self.pages = torch.zeros(n_q, hkv, max(k_pages, 1), device=dev, dtype=torch.int32)
            self.kmin = torch.empty(hkv, max(n_pages, 1), d, device=dev, dtype=kdt)
            self.kmax = torch.empty(hkv, max(n_pages, 1), d, device=dev, dtype=kdt)
            self.q_prev = torch.zeros(n_q, hq, d, device=dev, dtype=kdt)
            self.mse = torch.zeros(n_q, device=dev, dtype=torch.float64)
            self.active = torch.zeros(n_q, device=dev, dtype=torch.uint8)
            for name in ("a_res", "l_res", "pages", "kmin", "kmax", "q_prev", "mse", "active"):
                setattr(st, name, ptr(getattr(self, name)))
            # the selection as bitmaps: the refresh step's (residual mode) or
            # each step's own (reselect), read by the GATHER workgroups
            self.sel_bitmap = None
            if sel_bitmap:
                words = (max(n_pages, 1) + 31) // 32
                self.sel_bitmap = torch.zeros(n_q, hkv, words, device=dev, dtype=torch.int32)
                st.sel_bitmap = ptr(self.sel_bitmap)
            st.page_cap = n_pages if cache is not None else 0
            st.sparse_reselect = 1 if reselect else 0
        st.count_since_refresh = 1 if since_refresh else 0
        self.state = st
        self._dev = dev
        self.ws = None
        self._fit_workspace()

    def _fit_workspace(self):
        nbytes = max(fb_step_workspace(self.state), 16)
        if self.ws is None or self.ws.numel() < nbytes:
            self.ws = torch.empty(nbytes, device=self._dev, dtype=torch.uint8)
            self.state.ws, self.state.ws_bytes = ptr(self.ws), self.ws.numel()

    def next_block(self, k_blk, v_blk, stream=None):
        """Append the finished block's K/V to the cache and start the next block."""
        if self.cache is None:
            raise RuntimeError("next_block needs a Step built on a KVCache")
        fb_step_next_block(self.state, self.cache.cache, k_blk, v_blk, stream)
        self.k_prefix, self.v_prefix = self.cache.k_prefix, self.cache.v_prefix
        self._fit_workspace()

    @property
    def mask(self):
        """The [Hq] reuse flags the state holds (1 = reuse): in TEXT mode those
        the latest step used; in VIDEO mode, after a step, those the next step
        will use (the step swaps the flag buffers)."""
        cur = self.state.mask
        return self._masks[0] if self._masks[0].data_ptr() == cur else self._masks[1]

    @property
    def mask_next(self):
        cur = self.state.mask
        return self._masks[1] if self._masks[0].data_ptr() == cur else self._masks[0]

    def new_block(self):
        self.state.step = 0

    def step(self, q, k, v, a_full, l_full=None, ids=None, decision=-1, stream=None):
        args = fb_step_args()
        args.q_blk, args.k_blk, args.v_blk = tensors_of(self.shape, q, k, v)
        args.ids_cur = ptr(ids)
        args.decision = int(decision)
        args.a_full, args.l_full = ptr(a_full), ptr(l_full)
        fb_step(self.state, args, stream)
