"""ctypes mirror of include/flashblock.h and thin wrappers with the same names.

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream; every step of the computation
runs in libflashblock.so. Loading fails loudly when the library has not been
built: there is no fallback path.
"""

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashblock.so")

FB_OK, FB_ERR_INVALID_ARGUMENT, FB_ERR_UNSUPPORTED, FB_ERR_WORKSPACE_TOO_SMALL, FB_ERR_DEVICE = range(5)
FB_BF16, FB_F32 = 0, 1
FB_SEL_DENSE, FB_SEL_SPLIT, FB_SEL_GATHER = 0, 1, 2
FB_REUSE_COUNT, FB_REUSE_HEAD_COS, FB_REUSE_ACTIVE_MSE = 0, 1, 2
FB_STEP_TEXT, FB_STEP_VIDEO, FB_STEP_SPARSE = 0, 1, 2
ABI_VERSION = 3


class fb_attn_shape(C.Structure):
    _fields_ = [("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("scale", C.c_float), ("dtype", C.c_int)]


class fb_tensor(C.Structure):
    _fields_ = [("ptr", C.c_void_p), ("n_tok", C.c_int64),
                ("stride_tok", C.c_int64), ("stride_head", C.c_int64)]


class fb_page_sel(C.Structure):
    _fields_ = [("mode", C.c_int), ("page_size", C.c_int32), ("k_pages", C.c_int32),
                ("pages", C.c_void_p), ("active", C.c_void_p), ("bitmap", C.c_void_p)]


class fb_reuse_args(C.Structure):
    _fields_ = [("mode", C.c_int), ("n_q", C.c_int32), ("n_heads", C.c_int32),
                ("head_dim", C.c_int32),
                ("ids_prev", C.c_void_p), ("ids_cur", C.c_void_p), ("tau", C.c_int32),
                ("force", C.c_int32), ("m_count", C.c_void_p), ("ids_store", C.c_void_p),
                ("a_cached", C.c_void_p), ("a_probe", C.c_void_p), ("mask_in", C.c_void_p),
                ("gamma", C.c_double), ("sim", C.c_void_p),
                ("q_prev", C.c_void_p), ("q_cur", C.c_void_p), ("dtype", C.c_int),
                ("pct", C.c_int32), ("mse", C.c_void_p), ("active", C.c_void_p),
                ("mask", C.c_void_p), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("since_refresh", C.c_int32)]


class fb_kv_cache(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int64),
                ("n_tok", C.c_int64), ("stride_tok", C.c_int64), ("stride_head", C.c_int64)]


class fb_proxy_args(C.Structure):
    _fields_ = [("n_tok", C.c_int32), ("d_model", C.c_int32), ("rank", C.c_int32),
                ("dtype", C.c_int), ("x", C.c_void_p), ("x_stride", C.c_int64),
                ("factor", C.c_void_p), ("cache", C.c_void_p), ("n_select", C.c_int32),
                ("init", C.c_int32), ("sim", C.c_void_p), ("selected", C.c_void_p),
                ("mask", C.c_void_p), ("proxy", C.c_void_p), ("ws", C.c_void_p),
                ("ws_bytes", C.c_size_t)]


class fb_step_state(C.Structure):
    _fields_ = [("shape", fb_attn_shape), ("mode", C.c_int), ("n_q", C.c_int32),
                ("k_prefix", fb_tensor), ("v_prefix", fb_tensor),
                ("tau", C.c_int32), ("gamma", C.c_double), ("page_size", C.c_int32),
                ("k_pages", C.c_int32), ("pct", C.c_int32),
                ("a_out", C.c_void_p), ("l_out", C.c_void_p),
                ("a_probe", C.c_void_p), ("l_probe", C.c_void_p),
                ("a_res", C.c_void_p), ("l_res", C.c_void_p),
                ("ids_prev", C.c_void_p), ("m_count", C.c_void_p),
                ("mask", C.c_void_p), ("mask_next", C.c_void_p), ("sim", C.c_void_p),
                ("pages", C.c_void_p), ("kmin", C.c_void_p), ("kmax", C.c_void_p),
                ("q_prev", C.c_void_p), ("mse", C.c_void_p), ("active", C.c_void_p),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("step", C.c_int64), ("meta_ready", C.c_int32),
                ("page_cap", C.c_int64), ("count_since_refresh", C.c_int32),
                ("sparse_reselect", C.c_int32), ("sel_bitmap", C.c_void_p)]


class fb_step_args(C.Structure):
    _fields_ = [("q_blk", fb_tensor), ("k_blk", fb_tensor), ("v_blk", fb_tensor),
                ("ids_cur", C.c_void_p), ("decision", C.c_int32),
                ("a_full", C.c_void_p), ("l_full", C.c_void_p)]


# (name, restype, argtypes)
_SIGS = [
    ("fb_prefix_attn_workspace", C.c_size_t,
     [C.POINTER(fb_attn_shape), C.c_int64, C.c_int64, C.POINTER(fb_page_sel)]),
    ("fb_prefix_attn", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, fb_tensor, fb_tensor, C.c_void_p,
      C.POINTER(fb_page_sel), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
      C.c_void_p, C.c_size_t, C.c_void_p]),
    ("fb_prefix_attn_noalloc", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, fb_tensor, fb_tensor, C.c_void_p,
      C.POINTER(fb_page_sel), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    ("fb_block_attn_merge_workspace", C.c_size_t, [C.POINTER(fb_attn_shape), C.c_int64]),
    ("fb_block_attn_merge", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, fb_tensor, fb_tensor, C.c_void_p, C.c_void_p,
      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    ("fb_reuse_decide_workspace", C.c_size_t, [C.POINTER(fb_reuse_args)]),
    ("fb_reuse_decide", C.c_int, [C.POINTER(fb_reuse_args), C.c_void_p]),
    ("fb_page_meta", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]),
    ("fb_page_meta_update", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, C.c_int32, C.c_int64, C.c_int64, C.c_void_p,
      C.c_void_p, C.c_void_p]),
    ("fb_page_select_workspace", C.c_size_t, [C.POINTER(fb_attn_shape), C.c_int64, C.c_int64]),
    ("fb_page_select", C.c_int,
     [C.POINTER(fb_attn_shape), fb_tensor, C.c_void_p, C.c_void_p, C.c_int64, C.c_int64,
      C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    ("fb_page_bitmap", C.c_int,
     [C.POINTER(fb_attn_shape), C.c_void_p, C.c_int64, C.c_int64, C.c_int32, C.c_void_p,
      C.c_void_p]),
    ("fb_proxy_decide_workspace", C.c_size_t, [C.POINTER(fb_proxy_args)]),
    ("fb_proxy_decide", C.c_int, [C.POINTER(fb_proxy_args), C.c_void_p]),
    ("fb_layer_budgets", C.c_int,
     [C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_double, C.c_double, C.c_double,
      C.c_void_p, C.c_void_p]),
    ("fb_layer_taus", C.c_int,
     [C.c_int32, C.c_int32, C.c_int32, C.c_double, C.c_void_p, C.c_void_p]),
    ("fb_kv_append", C.c_int,
     [C.POINTER(fb_attn_shape), C.POINTER(fb_kv_cache), fb_tensor, fb_tensor, C.c_void_p]),
    ("fb_step_workspace", C.c_size_t, [C.POINTER(fb_step_state)]),
    ("fb_step", C.c_int, [C.POINTER(fb_step_state), C.POINTER(fb_step_args), C.c_void_p]),
    ("fb_step_next_block", C.c_int,
     [C.POINTER(fb_step_state), C.POINTER(fb_kv_cache), fb_tensor, fb_tensor, C.c_void_p]),
    ("fb_status_string", C.c_char_p, [C.c_int]),
    ("fb_abi_version", C.c_int, []),
]
SYMBOLS = [s[0] for s in _SIGS]

_lib = None


class FlashBlockError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))


def load(path=LIB_PATH):
    """Load libflashblock.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        if path != LIB_PATH and _lib._name != path:
            raise RuntimeError("another libflashblock is already loaded")
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libflashblock.so is not built (%s); run "
                           "`python -m block_diffusion_attention_amd.build`" % path)
    lib = C.CDLL(path)
    for name, res, args in _SIGS:
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.fb_abi_version() != ABI_VERSION:
        raise RuntimeError("ABI version mismatch")
    _lib = lib
    return lib


def status_string(status):
    return load().fb_status_string(int(status)).decode()


def _check(fn, status):
    if status != FB_OK:
        raise FlashBlockError(fn, status)


# ---------------------------------------------------------------- marshalling

def dtype_code(t):
    if t == torch.bfloat16:
        return FB_BF16
    if t == torch.float32:
        return FB_F32
    raise ValueError("unsupported dtype %s" % t)


def shape_of(n_q_heads, n_kv_heads, head_dim, scale, dtype):
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return fb_attn_shape(int(n_q_heads), int(n_kv_heads), int(head_dim), float(scale), code)


def tensor_of(t):
    """fb_tensor of a [n_tok, heads, d] tensor (any token/head strides, dim stride 1)."""
    if t is None:
        return fb_tensor(None, 0, 0, 0)
    if t.dim() != 3 or (t.shape[2] > 1 and t.stride(2) != 1):
        raise ValueError("expected [n_tok, heads, d] with contiguous d")
    ptr = t.data_ptr() if t.numel() else None
    return fb_tensor(ptr, t.shape[0], t.stride(0), t.stride(1))


def tensors_of(shape, q, k, v):
    """fb_tensors of q [n, Hq, d] and k, v [n_kv, Hkv, d], their head counts and
    widths checked against the shape first (the C calls see strides only, so a
    tensor of the wrong head count would be read as if it had the right one)."""
    for name, t, heads in (("q", q, shape.n_q_heads), ("k", k, shape.n_kv_heads),
                           ("v", v, shape.n_kv_heads)):
        if t is not None and t.dim() == 3 and (t.shape[1] != heads or t.shape[2] != shape.head_dim):
            raise ValueError("%s: expected [n, %d, %d], got %s"
                             % (name, heads, shape.head_dim, tuple(t.shape)))
    return tensor_of(q), tensor_of(k), tensor_of(v)


def ptr(t):
    return None if t is None else t.data_ptr()


def stream_of(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def page_sel(mode, page_size=16, pages=None, active=None, bitmap=None):
    k = 0 if pages is None else int(pages.shape[-1])
    return fb_page_sel(int(mode), int(page_size), k, ptr(pages), ptr(active), ptr(bitmap))


def fb_page_bitmap(shape, pages, n_pages, bitmap, stream=None):
    """Selection bitmaps [n_q, Hkv, ceil(n_pages / 32)] uint32 of page lists
    pages [n_q, Hkv, k]."""
    _check("fb_page_bitmap", load().fb_page_bitmap(
        C.byref(shape), ptr(pages), int(pages.shape[0]), int(n_pages), int(pages.shape[-1]),
        ptr(bitmap), stream_of(stream)))


# ------------------------------------------------------------------- wrappers

def fb_prefix_attn_workspace(shape, n_q, n_kv, sel=None):
    return load().fb_prefix_attn_workspace(C.byref(shape), int(n_q), int(n_kv),
                                           C.byref(sel) if sel is not None else None)


def fb_prefix_attn(shape, q, k, v, a_out, l_out, mask=None, sel=None, a_res=None,
                   l_res=None, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    tq, tk, tv = tensors_of(shape, q, k, v)
    st = load().fb_prefix_attn(C.byref(shape), tq, tk, tv,
                               ptr(mask), C.byref(sel) if sel is not None else None,
                               ptr(a_out), ptr(l_out), ptr(a_res), ptr(l_res), ptr(ws),
                               ws_bytes, stream_of(stream))
    _check("fb_prefix_attn", st)


NOALLOC_SCRATCH_BYTES = 16 << 20


def fb_prefix_attn_noalloc(shape, q, k, v, a_out, l_out, mask=None, sel=None, a_res=None,
                           l_res=None, stream=None):
    tq, tk, tv = tensors_of(shape, q, k, v)
    st = load().fb_prefix_attn_noalloc(C.byref(shape), tq, tk, tv,
                                       ptr(mask), C.byref(sel) if sel is not None else None,
                                       ptr(a_out), ptr(l_out), ptr(a_res), ptr(l_res),
                                       stream_of(stream))
    _check("fb_prefix_attn_noalloc", st)


def fb_block_attn_merge_workspace(shape, n_q):
    return load().fb_block_attn_merge_workspace(C.byref(shape), int(n_q))


def fb_block_attn_merge(shape, q, k, v, a_out, l_out, a_full, l_full=None, a_in=None,
                        l_in=None, ws=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    tq, tk, tv = tensors_of(shape, q, k, v)
    st = load().fb_block_attn_merge(C.byref(shape), tq, tk, tv,
                                    ptr(a_out), ptr(l_out), ptr(a_full), ptr(l_full),
                                    ptr(a_in), ptr(l_in), ptr(ws), ws_bytes, stream_of(stream))
    _check("fb_block_attn_merge", st)


def fb_reuse_decide_workspace(args):
    return load().fb_reuse_decide_workspace(C.byref(args))


def fb_reuse_decide(args, stream=None):
    _check("fb_reuse_decide", load().fb_reuse_decide(C.byref(args), stream_of(stream)))


def fb_page_meta(shape, k, page_size, kmin, kmax, stream=None):
    _check("fb_page_meta", load().fb_page_meta(C.byref(shape), tensor_of(k), int(page_size),
                                               ptr(kmin), ptr(kmax), stream_of(stream)))


def fb_page_select_workspace(shape, n_q, n_pages):
    return load().fb_page_select_workspace(C.byref(shape), int(n_q), int(n_pages))


def fb_page_meta_update(shape, k, page_size, n_tok_old, page_cap, kmin, kmax, stream=None):
    _check("fb_page_meta_update",
           load().fb_page_meta_update(C.byref(shape), tensor_of(k), int(page_size),
                                      int(n_tok_old), int(page_cap), ptr(kmin), ptr(kmax),
                                      stream_of(stream)))


def fb_page_select(shape, q, kmin, kmax, n_pages, k_pages, pages, bound=None, ws=None,
                   stream=None, page_cap=0, active=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().fb_page_select(C.byref(shape), tensor_of(q), ptr(kmin), ptr(kmax),
                               int(n_pages), int(page_cap), int(k_pages), ptr(active), ptr(pages),
                               ptr(bound), ptr(ws), ws_bytes, stream_of(stream))
    _check("fb_page_select", st)


def fb_proxy_decide_workspace(args):
    return load().fb_proxy_decide_workspace(C.byref(args))


def fb_proxy_decide(args, stream=None):
    _check("fb_proxy_decide", load().fb_proxy_decide(C.byref(args), stream_of(stream)))


def proxy_args(x, factor, cache, mask, selected=None, n_select=0, init=False, sim=None,
               proxy=None, ws=None):
    """fb_proxy_args of torch tensors: x [N, D], factor [D, r] (same dtype),
    cache [N, r] float64, mask [N] uint8, selected [n_select] int32."""
    if x.dim() != 2 or x.stride(1) != 1 or not factor.is_contiguous():
        raise ValueError("x must be [N, D] with contiguous rows, factor contiguous")
    a = fb_proxy_args()
    a.n_tok, a.d_model, a.rank = x.shape[0], x.shape[1], factor.shape[1]
    a.dtype = dtype_code(x.dtype)
    a.x, a.x_stride, a.factor = x.data_ptr(), x.stride(0), factor.data_ptr()
    a.cache, a.mask, a.selected = ptr(cache), ptr(mask), ptr(selected)
    a.n_select, a.init = int(n_select), 1 if init else 0
    a.sim, a.proxy = ptr(sim), ptr(proxy)
    a.ws, a.ws_bytes = ptr(ws), 0 if ws is None else ws.numel() * ws.element_size()
    return a


def fb_layer_taus(block, base_tau, mean_ratio, ratios):
    """Host schedule: per-layer reuse thresholds (list) from per-layer ratios."""
    n = len(ratios)
    r = (C.c_double * n)(*[float(x) for x in ratios])
    taus = (C.c_int32 * n)()
    _check("fb_layer_taus", load().fb_layer_taus(int(n), int(block), int(base_tau),
                                                 float(mean_ratio), r, taus))
    return list(taus)


def fb_layer_budgets(n_layers, n_tok, mean_ratio, floor_ratio, mu, s_left, s_right):
    """Host schedule: (ratios list, counts list) per layer."""
    ratios = (C.c_double * int(n_layers))()
    counts = (C.c_int32 * int(n_layers))()
    _check("fb_layer_budgets", load().fb_layer_budgets(
        int(n_layers), int(n_tok), float(mean_ratio), float(floor_ratio), float(mu),
        float(s_left), float(s_right), ratios, counts))
    return list(ratios), list(counts)


def fb_kv_append(shape, cache, k_blk, v_blk, stream=None):
    """cache: an fb_kv_cache (host struct; n_tok grows on success)."""
    _check("fb_kv_append", load().fb_kv_append(C.byref(shape), C.byref(cache), tensor_of(k_blk),
                                               tensor_of(v_blk), stream_of(stream)))


def fb_step_workspace(state):
    return load().fb_step_workspace(C.byref(state))


def fb_step(state, args, stream=None):
    _check("fb_step", load().fb_step(C.byref(state), C.byref(args), stream_of(stream)))


def fb_step_next_block(state, cache, k_blk, v_blk, stream=None):
    _check("fb_step_next_block",
           load().fb_step_next_block(C.byref(state), C.byref(cache), tensor_of(k_blk),
                                     tensor_of(v_blk), stream_of(stream)))


def fb_status_string(status):
    return status_string(status)


def fb_abi_version():
    return load().fb_abi_version()
