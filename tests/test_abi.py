"""Host-side checks of the C ABI that need no GPU: the built library loads and
exports every entry point the header declares, the ctypes structs match the
C layout, and invalid arguments are rejected with the documented status
before any HIP call."""

import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

import block_diffusion_attention_amd as fb
from block_diffusion_attention_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashblock.h")

FAKE = 0x7F0000100000          # aligned fake device address; never dereferenced


@pytest.fixture(scope="module")
def lib():
    return fb.load()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fb_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(_abi.SYMBOLS) == names


def test_status_strings_and_version(lib):
    assert fb.fb_abi_version() == 3
    assert fb.fb_status_string(0) == "ok"
    assert fb.fb_status_string(3) == "workspace too small"
    assert fb.fb_status_string(99) == "unknown status"


STRUCTS = {
    "fb_attn_shape": ["n_q_heads", "n_kv_heads", "head_dim", "scale", "dtype"],
    "fb_tensor": ["ptr", "n_tok", "stride_tok", "stride_head"],
    "fb_page_sel": ["mode", "page_size", "k_pages", "pages", "active", "bitmap"],
    "fb_reuse_args": [f[0] for f in _abi.fb_reuse_args._fields_],
    "fb_step_state": [f[0] for f in _abi.fb_step_state._fields_],
    "fb_step_args": [f[0] for f in _abi.fb_step_args._fields_],
    "fb_kv_cache": [f[0] for f in _abi.fb_kv_cache._fields_],
    "fb_proxy_args": [f[0] for f in _abi.fb_proxy_args._fields_],
}


def test_struct_layouts_match_c():
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "flashblock.h"', "int main(){"]
    for s, fields in STRUCTS.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (s, s))
        for f in fields:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (s, f, s, f))
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROOT, "include"),
                        "-I/opt/rocm/include", c, "-o", exe], check=True, capture_output=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    for s, fields in STRUCTS.items():
        cls = getattr(_abi, s)
        assert int(got[s]) == C.sizeof(cls), s
        for f in fields:
            assert int(got[s + "." + f]) == getattr(cls, f).offset, (s, f)


# ------------------------------------------------------- validation, no GPU

def shape(hq=32, hkv=8, d=128, dt=0, scale=0.088):
    return fb.fb_attn_shape(hq, hkv, d, scale, dt)


def ten(n, heads, d=128, st=None, sh=None, p=FAKE):
    st = heads * d if st is None else st
    sh = d if sh is None else sh
    return fb.fb_tensor(p, n, st, sh)


def prefix(lib, sh, q, k, v, a=FAKE, l=FAKE, sel=None, ar=None, lr=None, ws=None, wsb=0):
    return lib.fb_prefix_attn(C.byref(sh), q, k, v, None, C.byref(sel) if sel else None,
                              a, l, ar, lr, ws, wsb, None)


def test_prefix_rejects_bad_arguments(lib):
    q, k = ten(4, 32), ten(1000, 8)
    bad = fb.FB_ERR_INVALID_ARGUMENT
    assert prefix(lib, shape(hq=30), q, k, k) == bad                       # Hq % Hkv
    assert prefix(lib, shape(d=96), ten(4, 32, 96), ten(9, 8, 96), ten(9, 8, 96)) == fb.FB_ERR_UNSUPPORTED
    assert prefix(lib, shape(d=0), q, k, k) == bad
    assert prefix(lib, shape(scale=-1.0), q, k, k) == bad
    assert prefix(lib, shape(dt=7), q, k, k) == bad
    assert prefix(lib, shape(), ten(0, 32), k, k) == bad                   # n_q < 1
    assert prefix(lib, shape(), ten(4, 32, p=None), k, k) == bad            # NULL q
    assert prefix(lib, shape(), ten(4, 32, p=FAKE + 8), k, k) == bad        # misaligned
    assert prefix(lib, shape(), q, ten(1000, 8, st=1028), k) == bad        # stride % 8
    assert prefix(lib, shape(), q, ten(1000, 8, st=512, sh=128), k) == bad  # overlap
    assert prefix(lib, shape(), q, k, ten(999, 8)) == bad                   # |K| != |V|
    assert prefix(lib, shape(), q, k, k, a=None) == bad
    assert prefix(lib, shape(), q, k, k, ar=FAKE, lr=FAKE) == bad          # residual in dense
    sel = fb.fb_page_sel(fb.FB_SEL_SPLIT, 16, 10000, FAKE, None)
    assert prefix(lib, shape(), q, k, k, sel=sel, ar=FAKE, lr=FAKE) == bad  # k > pages
    sel = fb.fb_page_sel(fb.FB_SEL_SPLIT, 16, 8, FAKE, None)
    assert prefix(lib, shape(), q, k, k, sel=sel) == bad                    # residual missing


def test_prefix_workspace_rules(lib):
    sh = shape()
    q, k = ten(16, 32), ten(800000, 8)
    need = lib.fb_prefix_attn_workspace(C.byref(sh), 16, 800000, None)
    assert need > 0 and need % 256 == 0
    assert prefix(lib, sh, q, k, k, ws=FAKE, wsb=need - 1) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    assert prefix(lib, sh, q, k, k, ws=None, wsb=need) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    # a short prefix is one chunk written straight to the outputs
    assert lib.fb_prefix_attn_workspace(C.byref(sh), 4, 100, None) == 0
    # head-major K/V is accepted by the validator (workspace check is reached)
    kh = ten(800000, 8, st=128, sh=800000 * 128)
    assert prefix(lib, sh, q, kh, kh, ws=FAKE, wsb=need - 1) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    split = fb.fb_page_sel(fb.FB_SEL_SPLIT, 16, 819, FAKE, None)
    ns = lib.fb_prefix_attn_workspace(C.byref(sh), 8, 65536, C.byref(split))
    dense = lib.fb_prefix_attn_workspace(C.byref(sh), 8, 65536, None)
    assert ns > 0 and dense > 0


def test_block_merge_rejects(lib):
    sh = shape()
    q, k = ten(4, 32), ten(4, 8)
    f = lib.fb_block_attn_merge
    assert f(C.byref(sh), q, ten(5, 8), k, FAKE, FAKE, FAKE, None, None, None, None, 0, None) == 1
    assert f(C.byref(sh), q, k, k, None, FAKE, FAKE, None, None, None, None, 0, None) == 1
    assert f(C.byref(sh), q, k, k, FAKE, FAKE, None, None, None, None, None, 0, None) == 1


def test_reuse_decide_rejects(lib):
    a = fb.fb_reuse_args()
    a.mode, a.n_q, a.n_heads = fb.FB_REUSE_COUNT, 4, 32
    a.ids_cur, a.mask, a.force = FAKE, FAKE, 2
    assert lib.fb_reuse_decide(C.byref(a), None) == 1
    a.mode, a.force = fb.FB_REUSE_HEAD_COS, -1
    a.head_dim, a.a_cached, a.a_probe, a.sim = 128, FAKE, None, FAKE
    assert lib.fb_reuse_decide(C.byref(a), None) == 1
    a.a_probe = FAKE
    assert lib.fb_reuse_decide(C.byref(a), None) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    a.mode, a.q_prev, a.q_cur, a.active, a.pct = fb.FB_REUSE_ACTIVE_MSE, FAKE, FAKE, FAKE, 0
    assert lib.fb_reuse_decide(C.byref(a), None) == 1
    a.pct = 25
    assert lib.fb_reuse_decide_workspace(C.byref(a)) == 256
    assert lib.fb_reuse_decide(C.byref(a), None) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    a.mode = 9
    assert lib.fb_reuse_decide(C.byref(a), None) == 1


def test_page_calls_reject(lib):
    sh = shape()
    assert lib.fb_page_meta(C.byref(sh), ten(100, 8), 0, FAKE, FAKE, None) == 1
    assert lib.fb_page_select(C.byref(sh), ten(8, 32), FAKE, FAKE, 10, 0, 11, None, FAKE, FAKE,
                              None, 0, None) == 1
    assert lib.fb_page_select(C.byref(sh), ten(8, 32), FAKE, FAKE, 10, 0, 3, None, FAKE, None,
                              None, 0, None) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    # metadata storage smaller than the page count
    assert lib.fb_page_select(C.byref(sh), ten(8, 32), FAKE, FAKE, 10, 9, 3, None, FAKE, FAKE,
                              None, 0, None) == 1
    up = lib.fb_page_meta_update
    assert up(C.byref(sh), ten(100, 8), 16, 0, 6, FAKE, FAKE, None) == 1      # 7 pages > 6
    assert up(C.byref(sh), ten(100, 8), 16, 101, 7, FAKE, FAKE, None) == 1    # old > new
    assert up(C.byref(sh), ten(100, 8), 16, -1, 7, FAKE, FAKE, None) == 1
    assert up(C.byref(sh), ten(100, 8), 0, 0, 7, FAKE, FAKE, None) == 1       # page size
    assert up(C.byref(sh), ten(100, 8), 16, 0, 7, None, FAKE, None) == 1
    assert lib.fb_page_select_workspace(C.byref(sh), 8, 4096) == 8 * 8 * 4096 * 8


def test_step_rejects(lib):
    st = fb.fb_step_state()
    st.shape = shape()
    st.mode, st.n_q = fb.FB_STEP_TEXT, 4
    st.k_prefix = st.v_prefix = ten(1000, 8)
    st.a_out = st.l_out = st.mask = FAKE
    st.ws, st.ws_bytes = FAKE, 1 << 40
    args = fb.fb_step_args()
    args.q_blk, args.k_blk, args.v_blk = ten(4, 32), ten(4, 8), ten(4, 8)
    args.a_full, args.decision = FAKE, 3
    assert lib.fb_step(C.byref(st), C.byref(args), None) == 1            # bad decision
    args.decision = -1
    args.q_blk = ten(5, 32)
    assert lib.fb_step(C.byref(st), C.byref(args), None) == 1            # n_q mismatch
    args.q_blk = ten(4, 32)
    assert lib.fb_step(C.byref(st), C.byref(args), None) == 1            # ids missing
    # the block's tensors are checked before any launch of the step
    st.mode = fb.FB_STEP_VIDEO
    for bad in (dict(q_blk=ten(4, 32, p=FAKE + 8)), dict(k_blk=ten(3, 8)),
                dict(v_blk=ten(4, 8, st=8 * 128 + 4))):
        for k, v in bad.items():
            setattr(args, k, v)
        assert lib.fb_step(C.byref(st), C.byref(args), None) == 1, bad
        args.q_blk, args.k_blk, args.v_blk = ten(4, 32), ten(4, 8), ten(4, 8)
    st.mode = fb.FB_STEP_TEXT
    st.mode = 7
    assert lib.fb_step(C.byref(st), C.byref(args), None) == 1
    st.mode = fb.FB_STEP_TEXT
    st.k_prefix = st.v_prefix = ten(800000, 8)
    st.ws_bytes = 10
    assert lib.fb_step(C.byref(st), C.byref(args), None) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    assert lib.fb_step_workspace(C.byref(st)) > 0
    assert st.step == 0


def test_many_rows_merge_requires_aligned_outputs(lib):
    # 300 block tokens of a 12-head MHA model: the MFMA merge path (16-byte rows)
    sh = shape(hq=12, hkv=12)
    q, k = ten(300, 12), ten(300, 12)
    f = lib.fb_block_attn_merge
    args = (None, None, None, None, 0, None)
    assert f(C.byref(sh), q, k, k, FAKE + 4, FAKE, FAKE, *args) == 1            # a_out
    assert f(C.byref(sh), q, k, k, FAKE, FAKE, FAKE + 4, *args) == 1            # a_full
    assert f(C.byref(sh), q, k, k, FAKE, FAKE, FAKE, None, FAKE + 4, None, None, 0, None) == 1
    assert lib.fb_block_attn_merge_workspace(C.byref(sh), 300) == 0


def test_many_rows_prefix_workspace_covers_masked_split(lib):
    # a video-sized pass needs no partials unmasked, but a head mask splits the
    # keys into chunks, so the workspace holds their partials
    sh = shape(hq=12, hkv=12)
    need = lib.fb_prefix_attn_workspace(C.byref(sh), 4680, 12480, None)
    assert need >= 8 * 4680 * 12 * 129 * 4
    q, k = ten(4680, 12), ten(12480, 12)
    assert prefix(lib, sh, q, k, k, ws=FAKE, wsb=need - 1) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    # a short prefix has a single chunk and no workspace at all
    assert lib.fb_prefix_attn_workspace(C.byref(sh), 4680, 500, None) == 0


def test_page_select_rejects_counts_beyond_int32(lib):
    sh = shape()
    assert lib.fb_page_select(C.byref(sh), ten(8, 32), FAKE, FAKE, 1 << 31, 0, 3, None, FAKE, FAKE,
                              None, 0, None) == 1
    assert lib.fb_page_select(C.byref(sh), ten(8, 32), FAKE, FAKE, -1, 0, 0, None, FAKE, FAKE,
                              None, 0, None) == 1


def test_sparse_plan_workspace_includes_selection_buffers(lib):
    sh = shape()
    split = fb.fb_page_sel(fb.FB_SEL_SPLIT, 16, 819, FAKE, None)
    gather = fb.fb_page_sel(fb.FB_SEL_GATHER, 16, 819, FAKE, None)
    ns = lib.fb_prefix_attn_workspace(C.byref(sh), 8, 65536, C.byref(split))
    ng = lib.fb_prefix_attn_workspace(C.byref(sh), 8, 65536, C.byref(gather))
    bitmaps = 8 * 8 * (4096 // 32) * 4
    assert ns > bitmaps and ng > bitmaps + 8 * 4096 * 4           # GATHER adds the union list


def test_sparse_split_beyond_the_reduce_is_refused(lib):
    # 9,000,000 keys in 32-token pages: 281,250 pages fit the selection bitmap,
    # but at most 8,160 keys per chunk would need 1,103 split-K chunks, more
    # than the 1,024 the reduce merges: refused before any launch
    sh = shape()
    q = ten(8, 32)
    for mode in (fb.FB_SEL_SPLIT, fb.FB_SEL_GATHER):
        sel = fb.fb_page_sel(mode, 32, 64, FAKE, None)
        big = ten(9000000, 8)
        assert prefix(lib, sh, q, big, big, sel=sel, ar=FAKE, lr=FAKE, ws=FAKE,
                      wsb=1 << 40) == fb.FB_ERR_UNSUPPORTED
        # the largest prefix that fits (1,024 chunks of 8,160 keys) reaches the
        # workspace check instead
        edge = ten(1024 * 8160, 8)
        assert prefix(lib, sh, q, edge, edge, sel=sel, ar=FAKE, lr=FAKE, ws=FAKE,
                      wsb=0) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    st = fb.fb_step_state()
    st.shape = sh
    st.mode, st.n_q = fb.FB_STEP_SPARSE, 8
    st.k_prefix = st.v_prefix = ten(9000000, 8)
    st.a_out = st.l_out = st.mask = st.a_res = st.l_res = FAKE
    st.pages = st.kmin = st.kmax = st.q_prev = st.active = FAKE
    st.page_size, st.k_pages, st.pct = 32, 64, 25
    st.ws, st.ws_bytes = FAKE, 1 << 40
    args = fb.fb_step_args()
    args.q_blk, args.k_blk, args.v_blk = ten(8, 32), ten(8, 8), ten(8, 8)
    args.a_full, args.decision = FAKE, -1
    assert lib.fb_step(C.byref(st), C.byref(args), None) == fb.FB_ERR_UNSUPPORTED
    assert st.step == 0 and st.meta_ready == 0


def test_noalloc_prefix_refuses_beyond_its_scratch(lib):
    # checked before any HIP call: bad arguments, then the 16 MiB scratch limit
    assert fb.NOALLOC_SCRATCH_BYTES == 16 << 20
    sh = shape(hq=12, hkv=12)
    q, k = ten(4680, 12), ten(12480, 12)
    assert lib.fb_prefix_attn_workspace(C.byref(sh), 4680, 12480, None) > 16 << 20
    f = lib.fb_prefix_attn_noalloc
    assert f(C.byref(sh), q, k, k, None, None, FAKE, FAKE, None, None, None) == \
        fb.FB_ERR_WORKSPACE_TOO_SMALL
    assert f(C.byref(sh), q, k, k, None, None, None, FAKE, None, None, None) == \
        fb.FB_ERR_INVALID_ARGUMENT
    sel = fb.fb_page_sel(fb.FB_SEL_SPLIT, 32, 64, FAKE, None)
    big = ten(9000000, 8)
    assert f(C.byref(shape()), ten(8, 32), big, big, None, C.byref(sel), FAKE, FAKE, FAKE, FAKE,
             None) == fb.FB_ERR_UNSUPPORTED


def test_page_bitmap_rejects(lib):
    sh = shape()
    f = lib.fb_page_bitmap
    assert f(C.byref(sh), FAKE, 0, 4096, 819, FAKE, None) == 1        # n_q
    assert f(C.byref(sh), FAKE, 8, 0, 0, FAKE, None) == 1             # no pages
    assert f(C.byref(sh), FAKE, 8, 4096, 4097, FAKE, None) == 1       # k > pages
    assert f(C.byref(sh), None, 8, 4096, 3, FAKE, None) == 1          # pages NULL
    assert f(C.byref(sh), FAKE, 8, 4096, 3, None, None) == 1          # bitmap NULL
    assert f(C.byref(sh), FAKE, 8, 1 << 20, 3, FAKE, None) == fb.FB_ERR_UNSUPPORTED  # 32,768 words


# ------------------------------------------------------ growing cache, no GPU

def cache(cap=64, n=60, st=8 * 128, sh=128, k=FAKE, v=FAKE + (1 << 24)):
    return fb.fb_kv_cache(k, v, cap, n, st, sh)


def test_kv_append_rejects_and_leaves_the_count(lib):
    sh = shape()
    ap = lib.fb_kv_append
    c = cache()
    blk = ten(4, 8)
    assert ap(C.byref(sh), C.byref(c), blk, ten(5, 8), None) == 1        # |K| != |V|
    assert ap(C.byref(sh), C.byref(c), ten(5, 8), ten(5, 8), None) == 1  # 60 + 5 > 64
    assert ap(C.byref(sh), None, blk, blk, None) == 1
    c.n_tok = 65
    assert ap(C.byref(sh), C.byref(c), blk, blk, None) == 1              # n_tok > capacity
    c = cache(st=8 * 128 + 4)
    assert ap(C.byref(sh), C.byref(c), blk, blk, None) == 1              # stride % 8
    c = cache(st=512)
    assert ap(C.byref(sh), C.byref(c), blk, blk, None) == 1              # rows overlap
    c = cache(k=None)
    assert ap(C.byref(sh), C.byref(c), blk, blk, None) == 1              # NULL storage
    assert c.n_tok == 60
    c = cache()
    assert ap(C.byref(sh), C.byref(c), ten(0, 8), ten(0, 8), None) == 0  # empty block: no launch
    assert c.n_tok == 60


def test_step_next_block_requires_the_state_to_view_the_cache(lib):
    st = fb.fb_step_state()
    st.shape = shape()
    st.mode, st.n_q = fb.FB_STEP_TEXT, 4
    c = cache(n=40)
    st.k_prefix = fb.fb_tensor(c.k, 40, c.stride_tok, c.stride_head)
    st.v_prefix = fb.fb_tensor(c.v, 40, c.stride_tok, c.stride_head)
    st.step = 3
    nb = lib.fb_step_next_block
    blk = ten(4, 8)
    st.k_prefix.n_tok = 39
    assert nb(C.byref(st), C.byref(c), blk, blk, None) == 1              # counts differ
    st.k_prefix.n_tok = 40
    st.v_prefix = fb.fb_tensor(c.k, 40, c.stride_tok, c.stride_head)
    assert nb(C.byref(st), C.byref(c), blk, blk, None) == 1              # v views k storage
    st.v_prefix = fb.fb_tensor(c.v, 40, c.stride_tok, c.stride_head)
    assert nb(C.byref(st), C.byref(c), ten(30, 8), ten(30, 8), None) == 1  # beyond capacity
    st.mode, st.page_size, st.page_cap = fb.FB_STEP_SPARSE, 16, 2
    assert nb(C.byref(st), C.byref(c), blk, blk, None) == 1              # 3 pages > page_cap 2
    assert st.step == 3 and c.n_tok == 40 and st.k_prefix.n_tok == 40


# ------------------------------------------------------ proxy identifier, no GPU

def test_proxy_decide_rejects(lib):
    a = fb.fb_proxy_args()
    a.n_tok, a.d_model, a.rank, a.dtype = 1024, 4096, 128, fb.FB_BF16
    a.x, a.x_stride, a.factor, a.cache, a.mask = FAKE, 4096, FAKE, FAKE, FAKE
    a.n_select, a.selected = 256, FAKE
    need = lib.fb_proxy_decide_workspace(C.byref(a))
    # partials of 8 blocks of 512 + the proxies + the negated keys + the
    # selection words (16, one 256-byte aligned region)
    assert need == 8 * 1024 * 128 * 8 + 1024 * 128 * 8 + 1024 * 8 + 256
    assert lib.fb_proxy_decide(C.byref(a), None) == fb.FB_ERR_WORKSPACE_TOO_SMALL
    a.ws, a.ws_bytes = FAKE, need
    for field, bad, want in (("x_stride", 4095, 1), ("n_select", 1025, 1), ("n_select", -1, 1),
                             ("init", 2, 1), ("rank", 48, 2), ("rank", 160, 2), ("dtype", 5, 1),
                             ("n_tok", 0, 1), ("x", None, 1), ("selected", None, 1)):
        old = getattr(a, field)
        setattr(a, field, bad)
        assert lib.fb_proxy_decide(C.byref(a), None) == want, field
        setattr(a, field, old)
    a.init, a.selected = 1, None              # init: the selection is not used
    a.ws_bytes = need - 1
    assert lib.fb_proxy_decide(C.byref(a), None) == fb.FB_ERR_WORKSPACE_TOO_SMALL


def test_page_select_refuses_beyond_its_grid_and_lds(lib):
    sh = shape()
    # more block tokens than the bound grid's token tiles cover
    assert lib.fb_page_select(C.byref(sh), ten(70000, 32), FAKE, FAKE, 100, 0, 3, None, FAKE,
                              FAKE, None, 0, None) == 2
    # 64 query heads on one KV head at d = 128: one token's rows do not fit the
    # generic bound kernel's 64 KB with the page rows
    assert lib.fb_page_select(C.byref(shape(64, 1)), ten(4, 64), FAKE, FAKE, 100, 0, 3, None,
                              FAKE, FAKE, None, 0, None) == 2


def test_binding_checks_head_counts():
    """The C calls see strides only; the binding refuses tensors whose head
    count or width disagrees with the shape before calling them."""
    import torch
    sh = shape()
    q = torch.zeros(4, 32, 128, dtype=torch.bfloat16)
    k_ok = torch.zeros(100, 8, 128, dtype=torch.bfloat16)
    k_bad = torch.zeros(100, 32, 128, dtype=torch.bfloat16)
    a = torch.zeros(4, 32, 128)
    l = torch.zeros(4, 32)
    with pytest.raises(ValueError, match="k: expected"):
        fb.fb_prefix_attn(sh, q, k_bad, k_ok, a, l)
    with pytest.raises(ValueError, match="v: expected"):
        fb.fb_prefix_attn(sh, q, k_ok, k_bad, a, l)
    with pytest.raises(ValueError, match="q: expected"):
        fb.fb_prefix_attn(sh, torch.zeros(4, 8, 128, dtype=torch.bfloat16), k_ok, k_ok, a, l)
    with pytest.raises(ValueError, match="k: expected"):
        fb.fb_block_attn_merge(sh, q, torch.zeros(4, 32, 128, dtype=torch.bfloat16),
                               torch.zeros(4, 8, 128, dtype=torch.bfloat16), a, l, a)
    with pytest.raises(ValueError, match="q: expected"):
        fb.fb_prefix_attn_noalloc(sh, torch.zeros(4, 32, 64, dtype=torch.bfloat16), k_ok, k_ok,
                                  a, l)
