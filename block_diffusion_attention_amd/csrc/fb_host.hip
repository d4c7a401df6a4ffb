// fb_host.hip -- the C ABI (include/flashblock.h): argument validation,
// split-K planning and workspace sizing, and the launch order of one
// FlashBlock denoising step on the caller's stream.
//
// Nothing here allocates, synchronises or keeps global state; every
// decision the method takes per step (FlashBlock technical summary, s2
// "adaptive reuse strategies") is taken on the device and consumed there.
#include <math.h>
#include <string.h>

#include <mutex>

#include "fb_internal.h"

namespace fb {
hipError_t launch_fill_u8(uint8_t* p, int n, uint8_t v, hipStream_t s);
hipError_t launch_copy_rows(const void* src, int64_t st, int64_t sh, void* dst, int n_q, int hq,
                            int d, fb_dtype dt, hipStream_t s);
}  // namespace fb

using namespace fb;

namespace {

// Split-K planning. A launch should put several workgroups on each of the
// 256 CUs (8 XCDs x 32); chunks are at least a few tiles per wave long so the
// partials stay a small fraction of the K/V bytes.
#ifndef FB_PREFIX_TARGET_WGS
#define FB_PREFIX_TARGET_WGS 256
#endif
#ifndef FB_PREFIX_MIN_TILES
#define FB_PREFIX_MIN_TILES 16
#endif
#ifndef FB_PREFIX_SLAB_ROWS
#define FB_PREFIX_SLAB_ROWS 64    // 32: query rows in 32-row slabs (one MFMA row block each)
#endif
#ifndef FB_PREFIX_PAIR
#define FB_PREFIX_PAIR 1          // 64-row slabs use the row-split (wave pair) kernel
#endif
#ifndef FB_PREFIX_PAIR_SMALL
#define FB_PREFIX_PAIR_SMALL 1    // <= 32 rows per KV head on head-major K/V: pair kernel
#endif
#ifndef FB_PREFIX_HEADS_INNER
#define FB_PREFIX_HEADS_INNER 1   // token-major K/V: item order heads-inner (see run_prefix)
#endif
#ifndef FB_TEXT_DECIDE_IN_PASS
#define FB_TEXT_DECIDE_IN_PASS 1  // device-decided text steps: the pass counts, no count launch
#endif
#ifndef FB_ROWS_MIN_ROWS
#define FB_ROWS_MIN_ROWS 128      // query rows per KV head from which the many-rows kernel runs
#endif
#ifndef FB_ROWS_MIN_TILES
#define FB_ROWS_MIN_TILES 32      // 32-key tiles per chunk of the many-rows kernel
#endif
#ifndef FB_ROWS_MAX_DYN
#define FB_ROWS_MAX_DYN 8         // key chunks a masked many-rows pass may take
#endif
#ifndef FB_SPARSE_GATHER_OCC
#define FB_SPARSE_GATHER_OCC 1    // GATHER pass: workgroups per CU the split-K plan aims at
#endif
#ifndef FB_TEXT_FUSE_REDUCE
#define FB_TEXT_FUSE_REDUCE 1   // text and sparse steps: the in-block kernel merges the partials
#endif
constexpr int64_t kMaxChunks = 1024;      // the reduce keeps per-chunk weights in LDS
constexpr int64_t kTargetWorkgroups = FB_PREFIX_TARGET_WGS;  // per resident round (x occupancy)
constexpr int64_t kMinTilesMfma = FB_PREFIX_MIN_TILES;   // 32-token tiles per chunk (4 waves)
constexpr int64_t kMinTilesGeneric = 4;   // 64-token tiles per chunk
constexpr int64_t kMinTilesSparse = 8;    // 32-key tiles per chunk of the sparse MFMA pass
constexpr int kMaxBitmapWords = 16384;    // selection bitmap row built in 64 KB of LDS
constexpr size_t kAlign = 256;

enum Path { PATH_GENERIC = 0, PATH_MFMA = 1, PATH_ROWS = 2, PATH_SPARSE = 3 };

struct PrefixPlan {
  int path = PATH_GENERIC;
  int row_blocks = 1;
  int n_slabs = 1;
  int n_rtiles = 1;            // PATH_ROWS: row tiles per KV head
  int dyn_max = 0;             // PATH_ROWS: key chunks of a masked pass, at most
  int64_t n_tiles = 0;
  int n_chunks = 0;
  int64_t tiles_per_chunk = 0;
  bool direct = false;         // one chunk, written straight to the outputs
  int64_t rows = 0;            // n_q * Hq
  size_t off_l = 0, off_ra = 0, off_rl = 0, ws_bytes = 0;
  size_t off_bm = 0, off_ul = 0, off_uc = 0;   // PATH_SPARSE: bitmaps, union list, union sizes
  int words = 0;
  int64_t n_pages = 0;
  bool fits = true;            // false: more split-K chunks than the reduce's LDS holds
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// The MFMA kernels address 32 token rows of a tile as 32-bit byte offsets.
bool offsets32(const fb_tensor& t) { return t.stride_tok < (int64_t(1) << 25); }

fb_status check_shape(const fb_attn_shape* s) {
  if (!s) return FB_ERR_INVALID_ARGUMENT;
  if (s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
    return FB_ERR_INVALID_ARGUMENT;
  if (s->dtype != FB_BF16 && s->dtype != FB_F32) return FB_ERR_INVALID_ARGUMENT;
  if (!(s->scale > 0.f) || !isfinite(s->scale)) return FB_ERR_INVALID_ARGUMENT;
  if (s->head_dim < 1) return FB_ERR_INVALID_ARGUMENT;
  if (s->head_dim != 64 && s->head_dim != 128) return FB_ERR_UNSUPPORTED;
  return FB_OK;
}

// n_tok must equal `want` when want >= 0. Token/head grid must not overlap:
// either token-major (stride_head >= d, stride_tok >= heads*stride_head) or
// head-major (stride_tok >= d, stride_head >= n_tok*stride_tok).
fb_status check_tensor(const fb_tensor& t, int64_t want, int heads, int d) {
  if (t.n_tok < 0) return FB_ERR_INVALID_ARGUMENT;
  if (want >= 0 && t.n_tok != want) return FB_ERR_INVALID_ARGUMENT;
  if (t.n_tok == 0) return FB_OK;
  if (!t.ptr || !aligned16(t.ptr)) return FB_ERR_INVALID_ARGUMENT;
  if (t.stride_tok < 0 || t.stride_head < 0) return FB_ERR_INVALID_ARGUMENT;
  if (t.stride_tok % 8 != 0 || t.stride_head % 8 != 0) return FB_ERR_INVALID_ARGUMENT;
  const bool one_head = heads == 1, one_tok = t.n_tok == 1;
  const bool tok_major = (one_head || t.stride_head >= d) &&
                         (one_tok || t.stride_tok >= (one_head ? d : heads * t.stride_head));
  const bool head_major = (one_tok || t.stride_tok >= d) &&
                          (one_head || t.stride_head >= t.n_tok * t.stride_tok);
  if (!tok_major && !head_major) return FB_ERR_INVALID_ARGUMENT;
  return FB_OK;
}

fb_status check_sel(const fb_page_sel* sel, const fb_attn_shape& s, int64_t n_q, int64_t n_kv) {
  if (!sel || sel->mode == FB_SEL_DENSE) return FB_OK;
  if (sel->mode != FB_SEL_SPLIT && sel->mode != FB_SEL_GATHER) return FB_ERR_INVALID_ARGUMENT;
  if (sel->page_size < 1 || sel->k_pages < 0) return FB_ERR_INVALID_ARGUMENT;
  const int64_t n_pages = (n_kv + sel->page_size - 1) / sel->page_size;
  if (sel->k_pages > n_pages) return FB_ERR_INVALID_ARGUMENT;
  if (sel->k_pages > 0 && !sel->pages) return FB_ERR_INVALID_ARGUMENT;
  (void)s;
  (void)n_q;
  return FB_OK;
}

// kv_head_major: each KV head's keys are contiguous (stride_head >= n_kv
// stride_tok), which decides the decode kernel for <= 32 rows per KV head.
PrefixPlan plan_prefix(const fb_attn_shape& s, int64_t n_q, int64_t n_kv, const fb_page_sel* sel,
                       bool kv_head_major) {
  PrefixPlan pl;
  const int mode = sel ? sel->mode : FB_SEL_DENSE;
  const int G = s.n_q_heads / s.n_kv_heads;
  const int64_t group_rows = n_q * G;
  pl.rows = n_q * s.n_q_heads;
  pl.path = (s.dtype == FB_BF16 && s.head_dim == 128 && mode == FB_SEL_DENSE) ? PATH_MFMA
                                                                             : PATH_GENERIC;
  if (pl.path == PATH_MFMA && group_rows >= FB_ROWS_MIN_ROWS) pl.path = PATH_ROWS;
  if (mode != FB_SEL_DENSE) {
    pl.n_pages = (n_kv + sel->page_size - 1) / sel->page_size;
    pl.words = static_cast<int>((pl.n_pages + 31) / 32);
    if (s.dtype == FB_BF16 && s.head_dim == 128 && sel->page_size % 16 == 0 &&
        pl.words <= kMaxBitmapWords)
      pl.path = PATH_SPARSE;
  }
  const int tile = (pl.path == PATH_ROWS || pl.path == PATH_SPARSE) ? 32 : prefix_tile_tokens(pl.path);
  int64_t n_virt = mode == FB_SEL_GATHER ? static_cast<int64_t>(sel->k_pages) * sel->page_size : n_kv;
  if (pl.path == PATH_SPARSE && mode == FB_SEL_GATHER)   // the union may reach every page
    n_virt = pl.n_pages * sel->page_size;
  const int64_t n_tiles = (n_virt + tile - 1) / tile;
  int64_t wg_per_chunk;
  int64_t min_tiles;
  if (pl.path == PATH_MFMA) {
    // <= 32 rows: the 32-row kernel on token-major K/V, the pair kernel (one
    // row block of each pair idle) on head-major K/V -- each measured 1-2.5%
    // ahead of the other on its layout
    const bool small_pair = FB_PREFIX_PAIR_SMALL && kv_head_major;
    pl.row_blocks = ((group_rows <= 32 && !small_pair) || FB_PREFIX_SLAB_ROWS == 32) ? 1 : 2;
    pl.n_slabs = static_cast<int>((group_rows + 32 * pl.row_blocks - 1) / (32 * pl.row_blocks));
    if (pl.row_blocks == 2 && FB_PREFIX_PAIR) pl.row_blocks = 3;   // kernel selector
    wg_per_chunk = s.n_kv_heads * pl.n_slabs;
    min_tiles = kMinTilesMfma;
  } else if (pl.path == PATH_SPARSE) {
    pl.n_slabs = static_cast<int>((group_rows + 31) / 32);
    wg_per_chunk = s.n_kv_heads * pl.n_slabs;
    min_tiles = kMinTilesSparse;
  } else if (pl.path == PATH_ROWS) {
    pl.n_rtiles = static_cast<int>((group_rows + rows_tile_rows() - 1) / rows_tile_rows());
    wg_per_chunk = s.n_kv_heads * static_cast<int64_t>(pl.n_rtiles);
    min_tiles = FB_ROWS_MIN_TILES;
  } else {
    wg_per_chunk = pl.rows;
    min_tiles = kMinTilesGeneric;
  }
  if (n_tiles > 0) {
    const int64_t occ = pl.path == PATH_MFMA   ? prefix_mfma_occupancy(pl.row_blocks)
                        : pl.path == PATH_ROWS ? rows_occupancy()
                        : (pl.path == PATH_SPARSE && mode == FB_SEL_GATHER) ? FB_SPARSE_GATHER_OCC
                                               : 1;
    int64_t want = kTargetWorkgroups * occ / wg_per_chunk;
    if (want < 1) want = 1;
    if (want > kMaxChunks) want = kMaxChunks;
    int64_t cap = n_tiles / min_tiles;
    if (cap < 1) cap = 1;
    int64_t chunks = want < cap ? want : cap;
    if (pl.path == PATH_SPARSE) {                  // bounded union slice per chunk
      const int64_t lo = (n_tiles + sparse_max_tiles_per_chunk() - 1) / sparse_max_tiles_per_chunk();
      chunks = chunks > lo ? chunks : lo;
    }
    // the reduce (and the in-block kernel's merge) keep one weight per chunk
    // in LDS arrays of kMaxChunks entries: a longer split is refused
    if (chunks > kMaxChunks) pl.fits = false;
    pl.tiles_per_chunk = (n_tiles + chunks - 1) / chunks;
    pl.n_chunks = static_cast<int>((n_tiles + pl.tiles_per_chunk - 1) / pl.tiles_per_chunk);
    if (pl.path == PATH_ROWS) {
      // a head mask leaves fewer groups: the pass then splits the keys further
      int64_t dm = cap < FB_ROWS_MAX_DYN ? cap : FB_ROWS_MAX_DYN;
      pl.dyn_max = static_cast<int>(dm > pl.n_chunks ? dm : pl.n_chunks);
    }
  }
  pl.n_tiles = n_tiles;
  pl.direct = pl.n_chunks == 1 && mode == FB_SEL_DENSE;
  const int ws_chunks = pl.dyn_max > pl.n_chunks ? pl.dyn_max : pl.n_chunks;
  if ((!pl.direct || ws_chunks > 1) && pl.n_chunks > 0) {
    const size_t nc = static_cast<size_t>(ws_chunks);
    const size_t a_bytes = align_up(nc * pl.rows * s.head_dim * sizeof(float));
    const size_t l_bytes = align_up(nc * pl.rows * sizeof(float));
    pl.off_l = a_bytes;
    pl.ws_bytes = a_bytes + l_bytes;
    if (mode == FB_SEL_SPLIT) {
      pl.off_ra = pl.ws_bytes;
      pl.off_rl = pl.off_ra + a_bytes;
      pl.ws_bytes = pl.off_rl + l_bytes;
    }
  }
  if (pl.path == PATH_SPARSE) {
    pl.off_bm = pl.ws_bytes;
    pl.ws_bytes += align_up(static_cast<size_t>(n_q) * s.n_kv_heads * pl.words * sizeof(uint32_t));
    if (mode == FB_SEL_GATHER) {
      pl.off_ul = pl.ws_bytes;
      pl.ws_bytes += align_up(static_cast<size_t>(s.n_kv_heads) * pl.n_pages * sizeof(int32_t));
      pl.off_uc = pl.ws_bytes;
      pl.ws_bytes += align_up(static_cast<size_t>(s.n_kv_heads) * sizeof(int32_t));
    }
  }
  return pl;
}

// Workspace of a prefix pass whatever the K/V layout (the layout picks the
// decode kernel, whose split may differ).
size_t prefix_ws_bytes(const fb_attn_shape& s, int64_t n_q, int64_t n_kv, const fb_page_sel* sel) {
  const size_t a = plan_prefix(s, n_q, n_kv, sel, false).ws_bytes;
  const size_t b = plan_prefix(s, n_q, n_kv, sel, true).ws_bytes;
  return a > b ? a : b;
}

fb_status dev(hipError_t e) { return e == hipSuccess ? FB_OK : FB_ERR_DEVICE; }

// Extra work a step folds into a prefix pass: for a sparse GATHER step, the
// token classification inside the selection prep (am) and the q_prev <- q_cur
// copy inside the reduce (q_src -> q_dst); for a dense text step or a sparse
// GATHER step, the reduce itself handed to the in-block kernel (defer).
struct PrefixHooks {
  const ActiveFromMse* am;
  const void* q_src; int64_t q_st, q_sh;
  void* q_dst; int q_esize;
  ReduceParams* defer;          // dense pass: fill this and leave the reduce to the caller
  const TextDecide* decide;     // dense MFMA / generic pass: it takes the text decision
};

bool kv_head_major(const fb_attn_shape& s, const fb_tensor& k, const fb_tensor& v) {
  return s.n_kv_heads == 1 || ((k.n_tok <= 1 || k.stride_head >= k.n_tok * k.stride_tok) &&
                               (v.n_tok <= 1 || v.stride_head >= v.n_tok * v.stride_tok));
}

fb_status run_prefix(const fb_attn_shape& s, const fb_tensor& q, const fb_tensor& k,
                     const fb_tensor& v, const uint8_t* mask, const fb_page_sel* sel, float* a_out,
                     float* l_out, float* a_res, float* l_res, void* ws, size_t ws_bytes,
                     hipStream_t stream, const PrefixHooks* hooks = nullptr) {
  const int64_t n_q = q.n_tok, n_kv = k.n_tok;
  const int mode = sel ? sel->mode : FB_SEL_DENSE;
  const PrefixPlan pl = plan_prefix(s, n_q, n_kv, sel, kv_head_major(s, k, v));
  if (!pl.fits) return FB_ERR_UNSUPPORTED;
  if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) return FB_ERR_WORKSPACE_TOO_SMALL;
  if (pl.ws_bytes > 0 && !aligned16(ws)) return FB_ERR_INVALID_ARGUMENT;

  char* w = static_cast<char*>(ws);
  PrefixParams pp;
  memset(&pp, 0, sizeof(pp));
  pp.q = q.ptr;
  pp.q_st = q.stride_tok;
  pp.q_sh = q.stride_head;
  pp.k = k.ptr;
  pp.v = v.ptr;
  pp.kv_st = k.stride_tok;
  pp.kv_sh = k.stride_head;
  pp.n_kv = n_kv;
  pp.n_q = static_cast<int>(n_q);
  pp.hq = s.n_q_heads;
  pp.hkv = s.n_kv_heads;
  pp.group = s.n_q_heads / s.n_kv_heads;
  pp.scale_log2 = s.scale * kLog2e;
  pp.mask = mask;
  pp.tiles_per_chunk = pl.tiles_per_chunk;
  pp.n_chunks = pl.n_chunks;
  pp.n_slabs = pl.n_slabs;
  // token-major K/V ([N, Hkv, d]): the KV heads of one key range run side by
  // side (on the XCDs in turn), so the reads in flight cover whole token
  // rows rather than one head's 256-byte slice of each
  pp.heads_inner = FB_PREFIX_HEADS_INNER && !kv_head_major(s, k, v);
  pp.sel_mode = mode;
  if (mode != FB_SEL_DENSE) {
    pp.page_size = sel->page_size;
    pp.k_pages = sel->k_pages;
    pp.pages = sel->pages;
    pp.active = mode == FB_SEL_GATHER ? sel->active : nullptr;
  }
  // many rows with a head mask: key chunks from the mask, partials + reduce
  const bool dyn = pl.path == PATH_ROWS && mask && pl.dyn_max > 1;
  if (pl.direct && !dyn) {
    pp.out = RowOut{a_out, l_out, 0};
  } else {
    pp.out = RowOut{reinterpret_cast<float*>(w), reinterpret_cast<float*>(w + pl.off_l), pl.rows};
    if (mode == FB_SEL_SPLIT)
      pp.out_res = RowOut{reinterpret_cast<float*>(w + pl.off_ra),
                          reinterpret_cast<float*>(w + pl.off_rl), pl.rows};
  }
  // K and V share strides in the kernels
  if (v.stride_tok != k.stride_tok || v.stride_head != k.stride_head) return FB_ERR_UNSUPPORTED;
  if (pl.path != PATH_GENERIC && !offsets32(k)) return FB_ERR_UNSUPPORTED;

  if (hooks && (pl.n_chunks == 0 || pl.direct)) return FB_ERR_UNSUPPORTED;   // they ride on both
  if (hooks && hooks->decide) {
    if (mode != FB_SEL_DENSE || mask || (pl.path != PATH_MFMA && pl.path != PATH_GENERIC))
      return FB_ERR_UNSUPPORTED;
    pp.decide_on = 1;
    pp.decide = *hooks->decide;
  }
  if (pl.n_chunks > 0) {
    hipError_t e;
    if (pl.path == PATH_SPARSE) {
      uint32_t* bm = reinterpret_cast<uint32_t*>(w + pl.off_bm);
      const bool gather = mode == FB_SEL_GATHER;
      int32_t* ul = gather ? reinterpret_cast<int32_t*>(w + pl.off_ul) : nullptr;
      int32_t* uc = gather ? reinterpret_cast<int32_t*>(w + pl.off_uc) : nullptr;
      // (k_pages = 0: all-zero bitmaps, no list is read)
      if (sel->bitmap) {
        // the caller's bitmaps: no selection prep; a GATHER pass takes the
        // union (and, with a classification hook, the active set) itself
        bm = const_cast<uint32_t*>(sel->bitmap);
        e = hipSuccess;
        if (gather) {
          if (!gather_union_fits(static_cast<int>(n_q), pl.words)) {
            if (hooks && hooks->am) return FB_ERR_UNSUPPORTED;
            e = launch_sel_union(bm, sel->active, static_cast<int>(n_q), s.n_kv_heads, pl.words,
                                 ul, uc, static_cast<int>(pl.n_pages), stream);
          } else {
            pp.union_from_bitmap = 1;
            if (hooks && hooks->am) {
              if (!gather_classify_fits(static_cast<int>(n_q), s.n_q_heads)) return FB_ERR_UNSUPPORTED;
              pp.classify = 1;
              pp.am = *hooks->am;
            }
          }
        } else if (hooks && hooks->am) {
          return FB_ERR_UNSUPPORTED;
        }
      } else if (hooks && hooks->am) {
        if (!gather || !sel_prep_mse_fits(static_cast<int>(n_q), s.n_q_heads, pl.words))
          return FB_ERR_UNSUPPORTED;
        e = launch_sel_prep_mse(sel->pages, static_cast<int>(n_q), s.n_kv_heads, sel->k_pages,
                                pl.words, static_cast<int>(pl.n_pages), *hooks->am, bm, ul, uc,
                                stream);
      } else if (sel_prep_fits(static_cast<int>(n_q), pl.words)) {
        e = launch_sel_prep(sel->pages, static_cast<int>(n_q), s.n_kv_heads, sel->k_pages, pl.words,
                            static_cast<int>(pl.n_pages), sel->active, gather ? 1 : 0, bm, ul, uc,
                            stream);
      } else {
        e = launch_sel_bitmap(sel->pages, static_cast<int>(n_q) * s.n_kv_heads, sel->k_pages,
                              pl.words, static_cast<int>(pl.n_pages), bm, stream);
        if (e == hipSuccess && gather)
          e = launch_sel_union(bm, sel->active, static_cast<int>(n_q), s.n_kv_heads, pl.words, ul,
                               uc, static_cast<int>(pl.n_pages), stream);
      }
      if (e != hipSuccess) return FB_ERR_DEVICE;
      pp.bitmap = bm;
      pp.words = pl.words;
      pp.n_pages = pl.n_pages;
      pp.ulist = ul;
      pp.ucnt = uc;
      e = launch_prefix_sparse(pp, stream);
    } else if (pl.path == PATH_ROWS) {
      RowsParams rp;
      memset(&rp, 0, sizeof(rp));
      rp.q = q.ptr;
      rp.q_st = q.stride_tok;
      rp.q_sh = q.stride_head;
      rp.k = k.ptr;
      rp.v = v.ptr;
      rp.k_st = rp.v_st = k.stride_tok;
      rp.k_sh = rp.v_sh = k.stride_head;
      rp.n_kv = n_kv;
      rp.n_q = static_cast<int>(n_q);
      rp.hq = s.n_q_heads;
      rp.hkv = s.n_kv_heads;
      rp.group = pp.group;
      rp.scale_log2 = pp.scale_log2;
      rp.mask = mask;
      rp.n_rtiles = pl.n_rtiles;
      rp.tiles_per_chunk = pl.tiles_per_chunk;
      rp.n_chunks = pl.n_chunks;
      if (dyn) {
        rp.dyn = RowsDyn{1, pl.n_rtiles, s.n_kv_heads, pp.group, pl.dyn_max,
                         static_cast<int>(kTargetWorkgroups) * rows_occupancy(), pl.n_tiles};
        rp.n_chunks = pl.dyn_max;
        rp.tiles_per_chunk = 0;                    // (from the mask, on the device)
      }
      rp.n_items = s.n_kv_heads * rp.n_chunks * pl.n_rtiles;
      rp.out = pp.out;
      e = launch_rows(rp, stream);
    } else {
      e = pl.path == PATH_MFMA ? launch_prefix_mfma(pp, pl.row_blocks, stream)
                               : launch_prefix_generic(pp, s.dtype, s.head_dim, stream);
    }
    if (e != hipSuccess) return FB_ERR_DEVICE;
  }
  if (pl.direct && !dyn) return FB_OK;
  ReduceParams rp;
  memset(&rp, 0, sizeof(rp));
  rp.part_a = pp.out.a;
  rp.part_l = pp.out.l;
  rp.n_chunks = pl.n_chunks;
  if (dyn)
    rp.dyn = RowsDyn{1, pl.n_rtiles, s.n_kv_heads, pp.group, pl.dyn_max,
                     static_cast<int>(kTargetWorkgroups) * rows_occupancy(), pl.n_tiles};
  rp.rows = pl.rows;
  rp.hq = s.n_q_heads;
  rp.d = s.head_dim;
  rp.mask = hooks && hooks->decide ? hooks->decide->mask : mask;
  rp.a_out = a_out;
  rp.l_out = l_out;
  if (hooks && hooks->q_src) {
    rp.q_src = hooks->q_src;
    rp.q_st = hooks->q_st;
    rp.q_sh = hooks->q_sh;
    rp.q_dst = hooks->q_dst;
    rp.q_esize = hooks->q_esize;
  }
  if (mode == FB_SEL_SPLIT) {
    rp.part_ra = pp.out_res.a;
    rp.part_rl = pp.out_res.l;
    rp.a_res = a_res;
    rp.l_res = l_res;
  } else if (mode == FB_SEL_GATHER) {
    rp.active = sel->active;
    rp.res_a = a_res;
    rp.res_l = l_res;
  }
  if (hooks && hooks->defer) {
    if (mode == FB_SEL_SPLIT || dyn) return FB_ERR_UNSUPPORTED;
    *hooks->defer = rp;
    return FB_OK;
  }
  return dev(launch_prefix_reduce(rp, stream));
}

fb_status validate_prefix(const fb_attn_shape* shape, const fb_tensor& q, const fb_tensor& k,
                          const fb_tensor& v, const fb_page_sel* sel, const float* a_out,
                          const float* l_out, const float* a_res, const float* l_res) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  const int d = shape->head_dim;
  if (q.n_tok < 1) return FB_ERR_INVALID_ARGUMENT;
  if ((st = check_tensor(q, -1, shape->n_q_heads, d)) != FB_OK) return st;
  if ((st = check_tensor(k, -1, shape->n_kv_heads, d)) != FB_OK) return st;
  if ((st = check_tensor(v, k.n_tok, shape->n_kv_heads, d)) != FB_OK) return st;
  if (!a_out || !l_out || !aligned16(a_out)) return FB_ERR_INVALID_ARGUMENT;
  if (q.n_tok > INT32_MAX / shape->n_q_heads) return FB_ERR_INVALID_ARGUMENT;
  if ((st = check_sel(sel, *shape, q.n_tok, k.n_tok)) != FB_OK) return st;
  const int mode = sel ? sel->mode : FB_SEL_DENSE;
  if (mode == FB_SEL_DENSE && (a_res || l_res)) return FB_ERR_INVALID_ARGUMENT;
  if (mode == FB_SEL_SPLIT && (!a_res || !l_res)) return FB_ERR_INVALID_ARGUMENT;
  // GATHER: the cached residual, or none at all (both NULL)
  if (mode == FB_SEL_GATHER && (a_res == nullptr) != (l_res == nullptr))
    return FB_ERR_INVALID_ARGUMENT;
  return FB_OK;
}

// true when the in-block pass of n_q block queries takes the one-wave-per-row
// kernel (which can also merge a dense pass's split-K partials)
bool block_rows_path(const fb_attn_shape& s, int64_t n_q) {
  const int G = s.n_q_heads / s.n_kv_heads;
  return s.dtype == FB_BF16 && s.head_dim == 128 && n_q * G >= FB_ROWS_MIN_ROWS;
}
bool block_small_path(const fb_attn_shape& s, int64_t n_q) {
  return !block_rows_path(s, n_q) && n_q <= 65535;
}

// The text step's reference-id update, when the prefix pass took the
// decision (the in-block kernel runs after it and writes the ids).
struct IdsUpdate {
  const int32_t* cur; int32_t* store; int n; int keep_on_reuse;
  const TextDecide* decide;     // nullable: the decision is taken by the in-block kernel
};

fb_status block_merge(const fb_attn_shape* shape, const fb_tensor& q_blk, const fb_tensor& k_blk,
                      const fb_tensor& v_blk, const float* a_out, const float* l_out,
                      float* a_full, float* l_full, float* a_in, float* l_in,
                      const ReduceParams* fused, float* cache_a, float* cache_l, void* q_dst,
                      hipStream_t stream, const IdsUpdate* ids = nullptr) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  const int d = shape->head_dim;
  if (q_blk.n_tok < 1) return FB_ERR_INVALID_ARGUMENT;
  if ((st = check_tensor(q_blk, -1, shape->n_q_heads, d)) != FB_OK) return st;
  if ((st = check_tensor(k_blk, q_blk.n_tok, shape->n_kv_heads, d)) != FB_OK) return st;
  if ((st = check_tensor(v_blk, q_blk.n_tok, shape->n_kv_heads, d)) != FB_OK) return st;
  if (!a_out || !l_out || !a_full) return FB_ERR_INVALID_ARGUMENT;
  if (q_blk.n_tok > INT32_MAX / shape->n_q_heads) return FB_ERR_INVALID_ARGUMENT;
  const int G = shape->n_q_heads / shape->n_kv_heads;
  if ((fused || ids) && !block_small_path(*shape, q_blk.n_tok)) return FB_ERR_UNSUPPORTED;
  if (ids && !ids->decide && (!fused || !fused->mask)) return FB_ERR_UNSUPPORTED;
  if (block_rows_path(*shape, q_blk.n_tok)) {
    // many rows: MFMA pass with the merge in its epilogue (16-byte row access)
    if (!aligned16(a_out) || !aligned16(a_full) || (a_in && !aligned16(a_in)))
      return FB_ERR_INVALID_ARGUMENT;
    if (!offsets32(k_blk) || !offsets32(v_blk)) return FB_ERR_UNSUPPORTED;
    RowsParams rp;
    memset(&rp, 0, sizeof(rp));
    rp.q = q_blk.ptr;
    rp.q_st = q_blk.stride_tok;
    rp.q_sh = q_blk.stride_head;
    rp.k = k_blk.ptr;
    rp.v = v_blk.ptr;
    rp.k_st = k_blk.stride_tok;
    rp.k_sh = k_blk.stride_head;
    rp.v_st = v_blk.stride_tok;
    rp.v_sh = v_blk.stride_head;
    rp.n_kv = q_blk.n_tok;
    rp.n_q = static_cast<int>(q_blk.n_tok);
    rp.hq = shape->n_q_heads;
    rp.hkv = shape->n_kv_heads;
    rp.group = G;
    rp.scale_log2 = shape->scale * kLog2e;
    rp.n_rtiles = static_cast<int>((q_blk.n_tok * G + rows_tile_rows() - 1) / rows_tile_rows());
    rp.n_chunks = 1;
    rp.tiles_per_chunk = (q_blk.n_tok + 31) / 32;
    rp.n_items = shape->n_kv_heads * rp.n_rtiles;
    rp.out = RowOut{a_full, l_full, 0};
    rp.a_prev = a_out;
    rp.l_prev = l_out;
    rp.a_raw = a_in;
    rp.l_raw = l_in;
    return dev(launch_rows(rp, stream));
  }
  if (q_blk.n_tok > 65535) return FB_ERR_UNSUPPORTED;
  BlockParams bp;
  memset(&bp, 0, sizeof(bp));
  bp.q = q_blk.ptr;
  bp.q_st = q_blk.stride_tok;
  bp.q_sh = q_blk.stride_head;
  bp.k = k_blk.ptr;
  bp.v = v_blk.ptr;
  bp.k_st = k_blk.stride_tok;
  bp.k_sh = k_blk.stride_head;
  bp.v_st = v_blk.stride_tok;
  bp.v_sh = v_blk.stride_head;
  bp.n_q = static_cast<int>(q_blk.n_tok);
  bp.hq = shape->n_q_heads;
  bp.hkv = shape->n_kv_heads;
  bp.group = shape->n_q_heads / shape->n_kv_heads;
  bp.d = d;
  bp.scale_log2 = shape->scale * kLog2e;
  bp.a_out = a_out;
  bp.l_out = l_out;
  bp.a_full = a_full;
  bp.l_full = l_full;
  bp.a_in = a_in;
  bp.l_in = l_in;
  if (fused) {
    bp.part_a = fused->part_a;
    bp.part_l = fused->part_l;
    bp.n_chunks = fused->n_chunks;
    bp.rows = fused->rows;
    bp.mask = fused->mask;
    bp.active = fused->active;
    bp.res_a = fused->res_a;
    bp.res_l = fused->res_l;
    bp.cache_a = cache_a;
    bp.cache_l = cache_l;
  }
  bp.q_dst = q_dst;
  if (ids) {
    bp.ids_cur = ids->cur;
    bp.ids_store = ids->store;
    bp.ids_n = ids->n;
    bp.ids_keep_on_reuse = ids->keep_on_reuse;
    if (ids->decide) {
      bp.decide_on = 1;
      bp.decide = *ids->decide;
    }
  }
  return dev(launch_block_small(bp, shape->dtype, stream));
}

// ---------------------------------------------------------------------------
// Scratch for fb_prefix_attn_noalloc: the split-K partials (and, for sparse
// selections, the bitmaps and the page union) live in this fixed device
// array instead of a caller workspace. Each GPU the library runs on holds its
// own copy until the process ends. Its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and kept; host code
// never passes the array's name itself to a kernel or a copy.
constexpr size_t kScratchBytes = size_t(16) << 20;     // FB_NOALLOC_SCRATCH_BYTES
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

fb_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FB_ERR_DEVICE;
  if (dev >= kMaxDevices) return FB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FB_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FB_OK;
}

}  // namespace

extern "C" {

const char* fb_status_string(fb_status s) {
  switch (s) {
    case FB_OK: return "ok";
    case FB_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FB_ERR_UNSUPPORTED: return "unsupported configuration";
    case FB_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case FB_ERR_DEVICE: return "device (HIP) error";
  }
  return "unknown status";
}

int fb_abi_version(void) { return FB_ABI_VERSION; }

size_t fb_prefix_attn_workspace(const fb_attn_shape* shape, int64_t n_q, int64_t n_kv,
                                const fb_page_sel* sel) {
  if (check_shape(shape) != FB_OK || n_q < 1 || n_kv < 0) return 0;
  if (check_sel(sel, *shape, n_q, n_kv) != FB_OK) return 0;
  return prefix_ws_bytes(*shape, n_q, n_kv, sel);
}

fb_status fb_prefix_attn(const fb_attn_shape* shape, fb_tensor q, fb_tensor k, fb_tensor v,
                         const uint8_t* head_reuse_mask, const fb_page_sel* sel, float* a_out,
                         float* l_out, float* a_res, float* l_res, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  fb_status st = validate_prefix(shape, q, k, v, sel, a_out, l_out, a_res, l_res);
  if (st != FB_OK) return st;
  return run_prefix(*shape, q, k, v, head_reuse_mask, sel, a_out, l_out, a_res, l_res, ws,
                    ws_bytes, stream);
}

fb_status fb_prefix_attn_noalloc(const fb_attn_shape* shape, fb_tensor q, fb_tensor k,
                                 fb_tensor v, const uint8_t* head_reuse_mask,
                                 const fb_page_sel* sel, float* a_out, float* l_out,
                                 float* a_res, float* l_res, hipStream_t stream) {
  fb_status st = validate_prefix(shape, q, k, v, sel, a_out, l_out, a_res, l_res);
  if (st != FB_OK) return st;
  const PrefixPlan pl = plan_prefix(*shape, q.n_tok, k.n_tok, sel, kv_head_major(*shape, k, v));
  if (!pl.fits) return FB_ERR_UNSUPPORTED;
  if (pl.ws_bytes > kScratchBytes) return FB_ERR_WORKSPACE_TOO_SMALL;
  // the stream must run on the current device (whose scratch copy is used)
  int cur = -1;
  hipDevice_t sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess) return FB_ERR_DEVICE;
  if (stream && (hipStreamGetDevice(stream, &sdev) != hipSuccess)) return FB_ERR_DEVICE;
  if (stream && sdev != cur) return FB_ERR_INVALID_ARGUMENT;
  void* ws = nullptr;
  if (pl.ws_bytes > 0 && (st = scratch_of_current_device(&ws)) != FB_OK) return st;
  return run_prefix(*shape, q, k, v, head_reuse_mask, sel, a_out, l_out, a_res, l_res, ws,
                    pl.ws_bytes > 0 ? kScratchBytes : 0, stream);
}

size_t fb_block_attn_merge_workspace(const fb_attn_shape* shape, int64_t n_q) {
  (void)shape;
  (void)n_q;
  return 0;
}

fb_status fb_block_attn_merge(const fb_attn_shape* shape, fb_tensor q_blk, fb_tensor k_blk,
                              fb_tensor v_blk, const float* a_out, const float* l_out,
                              float* a_full, float* l_full, float* a_in, float* l_in, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return block_merge(shape, q_blk, k_blk, v_blk, a_out, l_out, a_full, l_full, a_in, l_in,
                     nullptr, nullptr, nullptr, nullptr, stream);
}

size_t fb_reuse_decide_workspace(const fb_reuse_args* a) {
  if (!a || a->n_q < 0 || a->n_heads < 1) return 0;
  switch (a->mode) {
    case FB_REUSE_COUNT: return 0;
    case FB_REUSE_HEAD_COS:
      return align_up(static_cast<size_t>(head_cos_chunks(a->n_q)) * a->n_heads * 3 * sizeof(double));
    case FB_REUSE_ACTIVE_MSE: return align_up(static_cast<size_t>(a->n_q) * sizeof(double));
  }
  return 0;
}

fb_status fb_reuse_decide(const fb_reuse_args* a, hipStream_t stream) {
  if (!a || a->n_heads < 1 || a->n_q < 0) return FB_ERR_INVALID_ARGUMENT;
  switch (a->mode) {
    case FB_REUSE_COUNT:
      if (!a->mask || (a->n_q > 0 && !a->ids_cur)) return FB_ERR_INVALID_ARGUMENT;
      if (a->force < -1 || a->force > 1) return FB_ERR_INVALID_ARGUMENT;
      if (a->since_refresh != 0 && a->since_refresh != 1) return FB_ERR_INVALID_ARGUMENT;
      return dev(launch_count(a->ids_prev, a->ids_cur, a->n_q, a->tau, a->force, a->n_heads,
                              a->mask, a->m_count, a->ids_store, a->since_refresh, stream));
    case FB_REUSE_HEAD_COS: {
      if (a->n_q < 1 || !a->a_cached || !a->a_probe || !a->sim || !a->mask)
        return FB_ERR_INVALID_ARGUMENT;
      if (a->head_dim < 1) return FB_ERR_INVALID_ARGUMENT;
      if (!isfinite(a->gamma)) return FB_ERR_INVALID_ARGUMENT;
      const size_t need = fb_reuse_decide_workspace(a);
      if (a->ws_bytes < need || !a->ws) return FB_ERR_WORKSPACE_TOO_SMALL;
      return dev(launch_head_cos(a->a_cached, a->a_probe, a->n_q, a->n_heads, a->head_dim,
                                 a->mask_in, a->gamma, a->sim, a->mask,
                                 static_cast<double*>(a->ws), head_cos_chunks(a->n_q), nullptr,
                                 nullptr, nullptr, stream));
    }
    case FB_REUSE_ACTIVE_MSE: {
      if (a->n_q < 1 || !a->q_prev || !a->q_cur || !a->active) return FB_ERR_INVALID_ARGUMENT;
      if (a->head_dim < 1 || a->pct < 1 || a->pct > 100) return FB_ERR_INVALID_ARGUMENT;
      if (a->dtype != FB_BF16 && a->dtype != FB_F32) return FB_ERR_INVALID_ARGUMENT;
      const size_t need = fb_reuse_decide_workspace(a);
      if (a->ws_bytes < need || !a->ws) return FB_ERR_WORKSPACE_TOO_SMALL;
      return dev(launch_active_mse(a->q_prev, a->q_cur, a->dtype, a->n_q, a->n_heads, a->head_dim,
                                   a->pct, a->mse, a->active, static_cast<double*>(a->ws),
                                   stream));
    }
  }
  return FB_ERR_INVALID_ARGUMENT;
}

fb_status fb_page_meta(const fb_attn_shape* shape, fb_tensor k, int32_t page_size, void* kmin,
                       void* kmax, hipStream_t stream) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  if ((st = check_tensor(k, -1, shape->n_kv_heads, shape->head_dim)) != FB_OK) return st;
  if (page_size < 1) return FB_ERR_INVALID_ARGUMENT;
  if (k.n_tok > 0 && (!kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)))
    return FB_ERR_INVALID_ARGUMENT;
  const int64_t n_pages = (k.n_tok + page_size - 1) / page_size;
  if (n_pages > INT32_MAX) return FB_ERR_UNSUPPORTED;
  return dev(launch_page_meta(k.ptr, k.stride_tok, k.stride_head, k.n_tok, shape->n_kv_heads,
                              shape->head_dim, page_size, shape->dtype, kmin, kmax, 0, n_pages,
                              n_pages, stream));
}

fb_status fb_page_meta_update(const fb_attn_shape* shape, fb_tensor k, int32_t page_size,
                              int64_t n_tok_old, int64_t page_cap, void* kmin, void* kmax,
                              hipStream_t stream) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  if ((st = check_tensor(k, -1, shape->n_kv_heads, shape->head_dim)) != FB_OK) return st;
  if (page_size < 1 || n_tok_old < 0 || n_tok_old > k.n_tok) return FB_ERR_INVALID_ARGUMENT;
  const int64_t n_pages = (k.n_tok + page_size - 1) / page_size;
  if (page_cap < n_pages) return FB_ERR_INVALID_ARGUMENT;
  if (n_pages > INT32_MAX) return FB_ERR_UNSUPPORTED;
  if (n_pages > 0 && (!kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)))
    return FB_ERR_INVALID_ARGUMENT;
  // pages wholly below n_tok_old keep their metadata; the old partial page
  // and every new page are recomputed
  return dev(launch_page_meta(k.ptr, k.stride_tok, k.stride_head, k.n_tok, shape->n_kv_heads,
                              shape->head_dim, page_size, shape->dtype, kmin, kmax,
                              n_tok_old / page_size, n_pages, page_cap, stream));
}

size_t fb_page_select_workspace(const fb_attn_shape* shape, int64_t n_q, int64_t n_pages) {
  if (check_shape(shape) != FB_OK || n_q < 1 || n_pages < 0) return 0;
  return align_up(static_cast<size_t>(n_q) * shape->n_kv_heads * n_pages * sizeof(double));
}

// fb_page_select, and (bitmap non-null, n_pages <= topk_bitmap_max()) the
// selection also written as bitmap words [n_q, Hkv, ceil(n_pages / 32)]
// for the active tokens' rows
static fb_status page_select_impl(const fb_attn_shape* shape, fb_tensor q, const void* kmin,
                                  const void* kmax, int64_t n_pages, int64_t page_cap,
                                  int32_t k_pages, const uint8_t* active, int32_t* pages,
                                  double* bound, uint32_t* bitmap, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  if (q.n_tok < 1 || q.n_tok > INT32_MAX / shape->n_q_heads) return FB_ERR_INVALID_ARGUMENT;
  if (q.n_tok > 65535) return FB_ERR_UNSUPPORTED;   // token tiles of the bound grid (<= 65,535)
  if ((st = check_tensor(q, -1, shape->n_q_heads, shape->head_dim)) != FB_OK) return st;
  if (n_pages < 0 || n_pages > INT32_MAX || k_pages < 0 || k_pages > n_pages)
    return FB_ERR_INVALID_ARGUMENT;
  if (n_pages > 0 && (!kmin || !kmax || !aligned16(kmin) || !aligned16(kmax)))
    return FB_ERR_INVALID_ARGUMENT;
  if (k_pages > 0 && !pages) return FB_ERR_INVALID_ARGUMENT;
  if (page_cap == 0) page_cap = n_pages;
  if (page_cap < n_pages) return FB_ERR_INVALID_ARGUMENT;
  const int G = shape->n_q_heads / shape->n_kv_heads;
  // the generic bound kernel (group sizes other than 1, 2, 4, 8) needs one
  // token's query rows and a page block's rows in 64 KB of LDS
  const bool g_kernel = G == 1 || G == 2 || G == 4 || G == 8;
  if (!g_kernel && page_bound_tokens(static_cast<int>(q.n_tok), G, shape->head_dim) < 1)
    return FB_ERR_UNSUPPORTED;
  if (!bound) {
    const size_t need = fb_page_select_workspace(shape, q.n_tok, n_pages);
    if (ws_bytes < need || (need > 0 && !ws)) return FB_ERR_WORKSPACE_TOO_SMALL;
    bound = static_cast<double*>(ws);
  }
  if (bitmap && n_pages > topk_bitmap_max()) return FB_ERR_UNSUPPORTED;
  return dev(launch_page_select(q.ptr, q.stride_tok, q.stride_head, kmin, kmax,
                                static_cast<int>(q.n_tok), shape->n_q_heads, shape->n_kv_heads,
                                shape->head_dim, n_pages, page_cap, k_pages, shape->dtype, active,
                                bound, pages, bitmap, stream));
}

fb_status fb_page_select(const fb_attn_shape* shape, fb_tensor q, const void* kmin,
                         const void* kmax, int64_t n_pages, int64_t page_cap, int32_t k_pages,
                         const uint8_t* active, int32_t* pages, double* bound, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return page_select_impl(shape, q, kmin, kmax, n_pages, page_cap, k_pages, active, pages, bound,
                          nullptr, ws, ws_bytes, stream);
}

fb_status fb_page_bitmap(const fb_attn_shape* shape, const int32_t* pages, int64_t n_q,
                         int64_t n_pages, int32_t k_pages, uint32_t* bitmap, hipStream_t stream) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  if (n_q < 1 || n_pages < 1 || n_pages > INT32_MAX || k_pages < 0 || k_pages > n_pages)
    return FB_ERR_INVALID_ARGUMENT;
  if (!bitmap || (k_pages > 0 && !pages)) return FB_ERR_INVALID_ARGUMENT;
  const int64_t words = (n_pages + 31) / 32;
  if (words > kMaxBitmapWords) return FB_ERR_UNSUPPORTED;
  if (n_q > INT32_MAX / shape->n_kv_heads) return FB_ERR_INVALID_ARGUMENT;
  return dev(launch_sel_bitmap(pages, static_cast<int>(n_q) * shape->n_kv_heads, k_pages,
                               static_cast<int>(words), static_cast<int>(n_pages), bitmap, stream));
}

size_t fb_proxy_decide_workspace(const fb_proxy_args* a) {
  if (!a || a->n_tok < 1 || a->d_model < 1 || !proxy_rank_ok(a->rank)) return 0;
  const size_t n = static_cast<size_t>(a->n_tok), r = static_cast<size_t>(a->rank);
  size_t ws = align_up(static_cast<size_t>(proxy_n_blocks(a->d_model)) * n * r * sizeof(double));
  if (!a->proxy) ws += align_up(n * r * sizeof(double));
  ws += align_up(n * sizeof(double));                 // negated keys (selection input)
  ws += align_up((n + 63) / 64 * sizeof(uint64_t));   // selection words, 64 tokens each
  return ws;
}

fb_status fb_proxy_decide(const fb_proxy_args* a, hipStream_t stream) {
  if (!a || a->n_tok < 1 || a->d_model < 1 || a->x_stride < a->d_model) return FB_ERR_INVALID_ARGUMENT;
  if (a->dtype != FB_BF16 && a->dtype != FB_F32) return FB_ERR_INVALID_ARGUMENT;
  if (!a->x || !a->factor || !a->cache || !a->mask || !aligned16(a->factor))
    return FB_ERR_INVALID_ARGUMENT;
  if (a->init != 0 && a->init != 1) return FB_ERR_INVALID_ARGUMENT;
  if (!a->init && (a->n_select < 0 || a->n_select > a->n_tok)) return FB_ERR_INVALID_ARGUMENT;
  if (!a->init && a->n_select > 0 && !a->selected) return FB_ERR_INVALID_ARGUMENT;
  if (!proxy_rank_ok(a->rank)) return FB_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(a->n_tok) * a->rank > INT32_MAX) return FB_ERR_UNSUPPORTED;
  const size_t need = fb_proxy_decide_workspace(a);
  if (a->ws_bytes < need || !a->ws) return FB_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(a->ws)) return FB_ERR_INVALID_ARGUMENT;
  const size_t n = static_cast<size_t>(a->n_tok), r = static_cast<size_t>(a->rank);
  const int nb = proxy_n_blocks(a->d_model);
  char* w = static_cast<char*>(a->ws);
  double* part = reinterpret_cast<double*>(w);
  w += align_up(static_cast<size_t>(nb) * n * r * sizeof(double));
  double* proxy = a->proxy;
  if (!proxy) {
    proxy = reinterpret_cast<double*>(w);
    w += align_up(n * r * sizeof(double));
  }
  double* neg_key = reinterpret_cast<double*>(w);
  w += align_up(n * sizeof(double));
  uint64_t* words = reinterpret_cast<uint64_t*>(w);
  fb_status rc = dev(launch_proxy_partials(a->x, a->x_stride, a->factor, a->dtype, a->n_tok,
                                           a->d_model, a->rank, part, stream));
  if (rc != FB_OK) return rc;
  rc = dev(launch_proxy_keys(part, nb, a->n_tok, a->rank, a->init, a->cache, proxy, a->sim,
                             neg_key, a->mask, stream));
  if (rc != FB_OK || a->init) return rc;
  if (a->n_select == 0) return dev(launch_fill_u8(a->mask, a->n_tok, 0, stream));
  // up to a few thousand tokens: rank counting (mask, cache rows, selection
  // words), then the ascending ids; beyond, the radix top-k and a scatter
  if (a->n_tok <= proxy_select_max_tok())
    return dev(launch_proxy_select(neg_key, a->n_tok, a->n_select, proxy, a->rank, a->cache,
                                   a->mask, words, a->selected, stream));
  // the lowest similarities are the largest negated ones (ties: lower id); the
  // top-k writes every token's mask byte
  rc = dev(launch_topk_rows(neg_key, 1, 1, a->n_tok, a->n_select, nullptr, a->selected, a->mask,
                            nullptr, stream));
  if (rc != FB_OK) return rc;
  return dev(launch_proxy_scatter(a->selected, a->n_select, a->n_tok, proxy, a->rank, a->cache,
                                  stream));
}

fb_status fb_layer_budgets(int32_t n_layers, int32_t n_tok, double mean_ratio, double floor_ratio,
                           double mu, double s_left, double s_right, double* ratios,
                           int32_t* counts) {
#pragma clang fp contract(off)
  if (n_layers < 1 || n_tok < 0 || !counts) return FB_ERR_INVALID_ARGUMENT;
  if (!isfinite(mean_ratio) || !isfinite(floor_ratio) || !isfinite(mu) || !isfinite(s_left) ||
      !isfinite(s_right))
    return FB_ERR_INVALID_ARGUMENT;
  if (!(s_left > 0.0) || !(s_right > 0.0)) return FB_ERR_INVALID_ARGUMENT;
  if (!(floor_ratio >= 0.0 && floor_ratio <= mean_ratio && mean_ratio <= 1.0))
    return FB_ERR_INVALID_ARGUMENT;
  // the same operations, in the same order, as the reference schedule
  double mg = 0.0;
  for (int l = 0; l < n_layers; ++l) {
    const double s = l < mu ? s_left : s_right;
    const double z = (l - mu) / s;
    mg = mg + exp(-0.5 * z * z);
  }
  mg = mg / n_layers;
  const double peak = floor_ratio + (mean_ratio - floor_ratio) / mg;
  for (int l = 0; l < n_layers; ++l) {
    const double s = l < mu ? s_left : s_right;
    const double z = (l - mu) / s;
    const double r = floor_ratio + (peak - floor_ratio) * exp(-0.5 * z * z);
    if (ratios) ratios[l] = r;
    double n = floor(r * n_tok + 0.5);
    n = n < 0.0 ? 0.0 : (n > n_tok ? n_tok : n);
    counts[l] = static_cast<int32_t>(n);
  }
  return FB_OK;
}

fb_status fb_layer_taus(int32_t n_layers, int32_t block, int32_t base_tau, double mean_ratio,
                        const double* ratios, int32_t* taus) {
#pragma clang fp contract(off)
  if (n_layers < 1 || block < 1 || base_tau < 1 || !ratios || !taus) return FB_ERR_INVALID_ARGUMENT;
  if (!isfinite(mean_ratio) || !(mean_ratio > 0.0 && mean_ratio <= 1.0))
    return FB_ERR_INVALID_ARGUMENT;
  for (int l = 0; l < n_layers; ++l)
    if (!isfinite(ratios[l])) return FB_ERR_INVALID_ARGUMENT;
  // tau_l = floor(base_tau mean_ratio / ratio_l + 1/2) in [1, block + 1];
  // a layer with no budget (ratio <= 0) never recomputes after its first step
  const double q = static_cast<double>(base_tau) * mean_ratio;
  const double never = static_cast<double>(block) + 1.0;
  for (int l = 0; l < n_layers; ++l) {
    double t = never;
    if (ratios[l] > 0.0) {
      t = floor(q / ratios[l] + 0.5);
      t = t < 1.0 ? 1.0 : (t > never ? never : t);
    }
    taus[l] = static_cast<int32_t>(t);
  }
  return FB_OK;
}

fb_status fb_kv_append(const fb_attn_shape* shape, fb_kv_cache* c, fb_tensor k_blk,
                       fb_tensor v_blk, hipStream_t stream) {
  fb_status st = check_shape(shape);
  if (st != FB_OK) return st;
  if (!c || c->capacity < 0 || c->n_tok < 0 || c->n_tok > c->capacity)
    return FB_ERR_INVALID_ARGUMENT;
  const int hkv = shape->n_kv_heads, d = shape->head_dim;
  if ((st = check_tensor(k_blk, -1, hkv, d)) != FB_OK) return st;
  if ((st = check_tensor(v_blk, k_blk.n_tok, hkv, d)) != FB_OK) return st;
  const int64_t b = k_blk.n_tok;
  if (b > c->capacity - c->n_tok) return FB_ERR_INVALID_ARGUMENT;
  if (b == 0) return FB_OK;
  if (b > INT32_MAX / hkv) return FB_ERR_INVALID_ARGUMENT;
  // the storage, as tensors over its whole capacity
  const fb_tensor ks = {c->k, c->capacity, c->stride_tok, c->stride_head};
  const fb_tensor vs = {c->v, c->capacity, c->stride_tok, c->stride_head};
  if ((st = check_tensor(ks, -1, hkv, d)) != FB_OK) return st;
  if ((st = check_tensor(vs, -1, hkv, d)) != FB_OK) return st;
  const int64_t es = shape->dtype == FB_BF16 ? 2 : 4;
  // a block already written at the cache's tail is not copied
  auto in_place = [&](const fb_tensor& t, const void* base) {
    return t.ptr == static_cast<const char*>(base) + c->n_tok * c->stride_tok * es &&
           t.stride_tok == c->stride_tok && t.stride_head == c->stride_head;
  };
  const void* k_src = in_place(k_blk, c->k) ? nullptr : k_blk.ptr;
  const void* v_src = in_place(v_blk, c->v) ? nullptr : v_blk.ptr;
  const fb_status rc =
      dev(launch_kv_append(k_src, k_blk.stride_tok * es, k_blk.stride_head * es, v_src,
                           v_blk.stride_tok * es, v_blk.stride_head * es, c->k, c->v,
                           c->stride_tok * es, c->stride_head * es, c->n_tok, static_cast<int>(b),
                           hkv, static_cast<int>(d * es), stream));
  if (rc != FB_OK) return rc;
  c->n_tok += b;
  return FB_OK;
}

// ---------------------------------------------------------------------------
// fb_step
// ---------------------------------------------------------------------------
size_t fb_step_workspace(const fb_step_state* st) {
  if (!st || check_shape(&st->shape) != FB_OK || st->n_q < 1) return 0;
  size_t ws = 0;
  fb_page_sel sel;
  memset(&sel, 0, sizeof(sel));
  const fb_page_sel* psel = nullptr;
  if (st->mode == FB_STEP_SPARSE) {
    sel.mode = FB_SEL_SPLIT;
    sel.page_size = st->page_size > 0 ? st->page_size : 1;
    sel.k_pages = st->k_pages;
    psel = &sel;
  }
  const size_t p1 = prefix_ws_bytes(st->shape, st->n_q, st->k_prefix.n_tok, psel);
  ws = p1;
  if (st->mode == FB_STEP_SPARSE && st->sparse_reselect) {   // dense first step
    const size_t p0 = prefix_ws_bytes(st->shape, st->n_q, st->k_prefix.n_tok, nullptr);
    ws = ws > p0 ? ws : p0;
  }
  if (st->mode == FB_STEP_SPARSE) {
    sel.mode = FB_SEL_GATHER;
    const size_t p2 = prefix_ws_bytes(st->shape, st->n_q, st->k_prefix.n_tok, &sel);
    const int64_t n_pages = (st->k_prefix.n_tok + sel.page_size - 1) / sel.page_size;
    const size_t p3 = fb_page_select_workspace(&st->shape, st->n_q, n_pages);
    const size_t p4 = align_up(static_cast<size_t>(st->n_q) * sizeof(double));
    ws = ws > p2 ? ws : p2;
    ws = ws > p3 ? ws : p3;
    ws = ws > p4 ? ws : p4;
  }
  if (st->mode == FB_STEP_VIDEO) {
    const size_t pc = align_up(static_cast<size_t>(head_cos_chunks(st->n_q)) * st->shape.n_q_heads *
                               3 * sizeof(double));
    ws = ws > pc ? ws : pc;
  }
  return ws;
}

fb_status fb_step(fb_step_state* st, const fb_step_args* a, hipStream_t stream) {
  if (!st || !a) return FB_ERR_INVALID_ARGUMENT;
  fb_status rc = check_shape(&st->shape);
  if (rc != FB_OK) return rc;
  const fb_attn_shape& s = st->shape;
  const int n_q = st->n_q, hq = s.n_q_heads, d = s.head_dim;
  if (n_q < 1 || a->q_blk.n_tok != n_q) return FB_ERR_INVALID_ARGUMENT;
  if (a->decision < -1 || a->decision > 1) return FB_ERR_INVALID_ARGUMENT;
  if (!st->a_out || !st->l_out || !st->mask || !a->a_full) return FB_ERR_INVALID_ARGUMENT;
  if ((rc = check_tensor(st->k_prefix, -1, s.n_kv_heads, d)) != FB_OK) return rc;
  if ((rc = check_tensor(st->v_prefix, st->k_prefix.n_tok, s.n_kv_heads, d)) != FB_OK) return rc;
  // the block's tensors too, before any launch of the step
  if ((rc = check_tensor(a->q_blk, n_q, hq, d)) != FB_OK) return rc;
  if ((rc = check_tensor(a->k_blk, n_q, s.n_kv_heads, d)) != FB_OK) return rc;
  if ((rc = check_tensor(a->v_blk, n_q, s.n_kv_heads, d)) != FB_OK) return rc;
  if (fb_step_workspace(st) > st->ws_bytes) return FB_ERR_WORKSPACE_TOO_SMALL;
  const bool first = st->step == 0;
  ReduceParams fused;                      // a pass's reduce left to the in-block kernel
  bool has_fused = false;
  void* q_dst = nullptr;                   // the in-block kernel's query copy (sparse steps)

  switch (st->mode) {
    case FB_STEP_TEXT: {
      if (!a->ids_cur || !st->ids_prev) return FB_ERR_INVALID_ARGUMENT;
      const int force = first ? 0 : a->decision;
      if (st->count_since_refresh != 0 && st->count_since_refresh != 1)
        return FB_ERR_INVALID_ARGUMENT;
      // with split-K partials and the one-wave in-block kernel, that kernel
      // merges the partials itself (no reduce launch); a step the device
      // decides then also lets the pass take the decision (no count launch)
      // and the in-block kernel update the reference ids
      const PrefixPlan pl = plan_prefix(s, n_q, st->k_prefix.n_tok, nullptr,
                                        kv_head_major(s, st->k_prefix, st->v_prefix));
      const bool fuse = FB_TEXT_FUSE_REDUCE && (pl.path == PATH_MFMA || pl.path == PATH_GENERIC) &&
                        !pl.direct && pl.n_chunks > 0 && block_small_path(s, n_q);
      if (fuse && force != 1 && FB_TEXT_DECIDE_IN_PASS) {
        rc = validate_prefix(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, st->a_out,
                             st->l_out, nullptr, nullptr);
        if (rc != FB_OK) return rc;
        const TextDecide td = {first ? nullptr : st->ids_prev, a->ids_cur, n_q, st->tau, force, hq,
                               st->mask, st->m_count};
        PrefixHooks hk;
        memset(&hk, 0, sizeof(hk));
        hk.defer = &fused;
        hk.decide = &td;
        rc = run_prefix(s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, nullptr, st->a_out,
                        st->l_out, nullptr, nullptr, st->ws, st->ws_bytes, stream, &hk);
        if (rc != FB_OK) return rc;
        const IdsUpdate ids = {a->ids_cur, st->ids_prev, n_q, st->count_since_refresh, nullptr};
        rc = block_merge(&s, a->q_blk, a->k_blk, a->v_blk, st->a_out, st->l_out, a->a_full,
                         a->l_full, nullptr, nullptr, &fused, st->a_out, st->l_out, nullptr, stream,
                         &ids);
        if (rc != FB_OK) return rc;
        st->step += 1;
        return FB_OK;
      }
      if (force == 1 && block_small_path(s, n_q) && FB_TEXT_DECIDE_IN_PASS) {
        // forced reuse: no pass; the in-block kernel counts and decides
        const TextDecide td = {st->ids_prev, a->ids_cur, n_q, st->tau, 1, hq, st->mask,
                               st->m_count};
        const IdsUpdate ids = {a->ids_cur, st->ids_prev, n_q, st->count_since_refresh, &td};
        rc = block_merge(&s, a->q_blk, a->k_blk, a->v_blk, st->a_out, st->l_out, a->a_full,
                         a->l_full, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, stream,
                         &ids);
        if (rc != FB_OK) return rc;
        st->step += 1;
        return FB_OK;
      }
      rc = dev(launch_count(first ? nullptr : st->ids_prev, a->ids_cur, n_q, st->tau, force, hq,
                            st->mask, st->m_count, st->ids_prev, st->count_since_refresh,
                            stream));
      if (rc != FB_OK) return rc;
      if (force != 1) {
        if (fuse) {
          rc = validate_prefix(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, st->a_out,
                               st->l_out, nullptr, nullptr);
          if (rc != FB_OK) return rc;
          PrefixHooks hk;
          memset(&hk, 0, sizeof(hk));
          hk.defer = &fused;
          rc = run_prefix(s, a->q_blk, st->k_prefix, st->v_prefix, st->mask, nullptr, st->a_out,
                          st->l_out, nullptr, nullptr, st->ws, st->ws_bytes, stream, &hk);
          if (rc != FB_OK) return rc;
          has_fused = true;
        } else {
          rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, st->mask, nullptr,
                              st->a_out, st->l_out, nullptr, nullptr, st->ws, st->ws_bytes, stream);
          if (rc != FB_OK) return rc;
        }
      }
      break;
    }
    case FB_STEP_VIDEO: {
      if (!st->a_probe || !st->l_probe || !st->mask_next || !st->sim) return FB_ERR_INVALID_ARGUMENT;
      if (first) {
        rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, nullptr, st->a_out,
                            st->l_out, nullptr, nullptr, st->ws, st->ws_bytes, stream);
        if (rc != FB_OK) return rc;
        rc = dev(launch_fill_u8(st->mask, hq, 0, stream));
        if (rc != FB_OK) return rc;
      } else if (a->decision != 1) {
        const uint8_t* used = a->decision == 0 ? nullptr : st->mask;
        rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, used, nullptr, st->a_probe,
                            st->l_probe, nullptr, nullptr, st->ws, st->ws_bytes, stream);
        if (rc != FB_OK) return rc;
        // the cosine against the cache, and the cache taking the probe's
        // pair for the heads recomputed, in one pass over both
        rc = dev(launch_head_cos(st->a_out, st->a_probe, n_q, hq, d, used, st->gamma, st->sim,
                                 st->mask_next, static_cast<double*>(st->ws), head_cos_chunks(n_q),
                                 st->a_out, st->l_probe, st->l_out, stream));
        if (rc != FB_OK) return rc;
        uint8_t* tmp = st->mask;
        st->mask = st->mask_next;
        st->mask_next = tmp;
      }
      break;
    }
    case FB_STEP_SPARSE: {
      if (st->sparse_reselect != 0 && st->sparse_reselect != 1) return FB_ERR_INVALID_ARGUMENT;
      const bool reselect = st->sparse_reselect == 1;
      if ((!reselect && (!st->a_res || !st->l_res)) || !st->pages || !st->kmin || !st->kmax ||
          !st->q_prev || !aligned16(st->q_prev) || !st->active)
        return FB_ERR_INVALID_ARGUMENT;
      if (st->page_size < 1 || st->pct < 1 || st->pct > 100) return FB_ERR_INVALID_ARGUMENT;
      const int64_t n_pages = (st->k_prefix.n_tok + st->page_size - 1) / st->page_size;
      if (st->k_pages < 0 || st->k_pages > n_pages) return FB_ERR_INVALID_ARGUMENT;
      if (st->page_cap < 0 || (st->page_cap > 0 && st->page_cap < n_pages))
        return FB_ERR_INVALID_ARGUMENT;
      const int64_t page_cap = st->page_cap > 0 ? st->page_cap : n_pages;
      fb_page_sel sel;
      memset(&sel, 0, sizeof(sel));
      sel.page_size = st->page_size;
      sel.k_pages = st->k_pages;
      sel.pages = st->pages;
      // a split the reduce cannot merge is refused before any launch
      for (fb_sel_mode m : {FB_SEL_SPLIT, FB_SEL_GATHER}) {
        sel.mode = m;
        if (!plan_prefix(s, n_q, st->k_prefix.n_tok, &sel, false).fits ||
            !plan_prefix(s, n_q, st->k_prefix.n_tok, &sel, true).fits)
          return FB_ERR_UNSUPPORTED;
      }
      sel.mode = FB_SEL_DENSE;
      // the step's token bookkeeping: active flags (query MSE, mode 1, or a
      // constant, mode 0), then q_prev <- q_cur; one kernel for text-sized
      // blocks, else separate kernels (whose MSE reads contiguous queries)
      auto token_step = [&](int mode, uint8_t fill) -> fb_status {
        if (active_step_fits(n_q, hq))
          return dev(launch_active_step(st->q_prev, a->q_blk.ptr, a->q_blk.stride_tok,
                                        a->q_blk.stride_head, s.dtype, n_q, hq, d, mode, fill,
                                        st->pct, st->mse, st->active, stream));
        fb_status r;
        if (mode == 1) {
          if (a->q_blk.stride_head != d || a->q_blk.stride_tok != static_cast<int64_t>(hq) * d)
            return FB_ERR_UNSUPPORTED;
          r = dev(launch_active_mse(st->q_prev, a->q_blk.ptr, s.dtype, n_q, hq, d, st->pct,
                                    st->mse, st->active, static_cast<double*>(st->ws), stream));
        } else {
          r = dev(launch_fill_u8(st->active, n_q, fill, stream));
        }
        if (r != FB_OK) return r;
        return dev(launch_copy_rows(a->q_blk.ptr, a->q_blk.stride_tok, a->q_blk.stride_head,
                                    st->q_prev, n_q, hq, d, s.dtype, stream));
      };
      // FlashBlock's residual mode with a bitmap buffer: the refresh step
      // writes the selection as bitmaps, later steps read them (no prep)
      const bool prebuilt = st->sel_bitmap != nullptr && !reselect &&
                            (n_pages + 31) / 32 <= kMaxBitmapWords;
      // a FlashBlock step the controller left open (decision -1) on the sparse
      // kernel: the token classification rides on the selection prep, or on
      // the GATHER pass itself when the bitmaps are prebuilt
      bool fuse_mse = false;
      if (!first && a->decision == -1 && !reselect && st->k_prefix.n_tok > 0) {
        fb_page_sel g = sel;
        g.mode = FB_SEL_GATHER;
        g.active = st->active;
        const PrefixPlan gp = plan_prefix(s, n_q, st->k_prefix.n_tok, &g, false);
        fuse_mse = gp.path == PATH_SPARSE && gp.n_chunks > 0 &&
                   (prebuilt ? gather_union_fits(static_cast<int>(n_q), gp.words) &&
                                   gather_classify_fits(static_cast<int>(n_q), hq)
                             : sel_prep_mse_fits(static_cast<int>(n_q), hq, gp.words));
      }
      if (first) {
        if (!st->meta_ready) {
          rc = fb_page_meta_update(&s, st->k_prefix, st->page_size, 0, page_cap, st->kmin,
                                   st->kmax, stream);
          if (rc != FB_OK) return rc;
          st->meta_ready = 1;
        }
        if (reselect) {
          // LoSA: a dense first step; pages are chosen at every later step
          rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, nullptr,
                              st->a_out, st->l_out, nullptr, nullptr, st->ws, st->ws_bytes,
                              stream);
        } else {
          rc = fb_page_select(&s, a->q_blk, st->kmin, st->kmax, n_pages, page_cap, st->k_pages,
                              nullptr, st->pages, nullptr, st->ws, st->ws_bytes, stream);
          if (rc != FB_OK) return rc;
          if (prebuilt && n_pages > 0) {
            rc = fb_page_bitmap(&s, st->pages, n_q, n_pages, st->k_pages, st->sel_bitmap, stream);
            if (rc != FB_OK) return rc;
            sel.bitmap = st->sel_bitmap;
          }
          sel.mode = FB_SEL_SPLIT;
          rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, &sel, st->a_out,
                              st->l_out, st->a_res, st->l_res, st->ws, st->ws_bytes, stream);
        }
        if (rc != FB_OK) return rc;
        rc = token_step(0, 1);                     // every token active at the refresh step
        if (rc != FB_OK) return rc;
      } else if (fuse_mse) {
        // one launch fewer: the selection prep classifies the tokens (query
        // MSE, cutoff, active flags) and the reduce copies q_cur to q_prev
        const ActiveFromMse am = {st->q_prev, a->q_blk.ptr, a->q_blk.stride_tok,
                                  a->q_blk.stride_head, s.dtype, hq, d, st->pct, st->mse,
                                  st->active};
        // and, with the one-wave in-block kernel, that kernel merges the
        // partials and copies the queries: no reduce launch
        PrefixHooks hk = {&am, a->q_blk.ptr, a->q_blk.stride_tok, a->q_blk.stride_head,
                          st->q_prev, s.dtype == FB_BF16 ? 2 : 4, nullptr};
        if (FB_TEXT_FUSE_REDUCE && block_small_path(s, n_q)) {
          hk.q_src = nullptr;
          hk.q_dst = nullptr;
          hk.defer = &fused;
          has_fused = true;
          q_dst = st->q_prev;
        }
        sel.mode = FB_SEL_GATHER;
        sel.active = st->active;
        if (prebuilt) sel.bitmap = st->sel_bitmap;
        rc = validate_prefix(&s, a->q_blk, st->k_prefix, st->v_prefix, &sel, st->a_out, st->l_out,
                             st->a_res, st->l_res);
        if (rc != FB_OK) return rc;
        rc = run_prefix(s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, &sel, st->a_out,
                        st->l_out, st->a_res, st->l_res, st->ws, st->ws_bytes, stream, &hk);
        if (rc != FB_OK) return rc;
      } else if (a->decision != 1) {
        rc = token_step(a->decision == 0 ? 0 : 1, 1);
        if (rc != FB_OK) return rc;
        // the active tokens' queries choose pages; with a bitmap buffer the
        // top-k also writes them as bitmaps and the GATHER workgroups take
        // their union themselves (no selection-prep launch)
        const bool sel_bits = reselect && st->sel_bitmap && st->k_pages > 0 &&
                              n_pages <= topk_bitmap_max() &&
                              gather_union_fits(static_cast<int>(n_q),
                                                static_cast<int>((n_pages + 31) / 32));
        if (reselect) {
          rc = page_select_impl(&s, a->q_blk, st->kmin, st->kmax, n_pages, page_cap, st->k_pages,
                                st->active, st->pages, nullptr, sel_bits ? st->sel_bitmap : nullptr,
                                st->ws, st->ws_bytes, stream);
          if (rc != FB_OK) return rc;
        }
        sel.mode = FB_SEL_GATHER;
        sel.active = st->active;
        if (prebuilt || sel_bits) sel.bitmap = st->sel_bitmap;
        float* ar = reselect ? nullptr : st->a_res;
        float* lr = reselect ? nullptr : st->l_res;
        const PrefixPlan gp = plan_prefix(s, n_q, st->k_prefix.n_tok, &sel,
                                          kv_head_major(s, st->k_prefix, st->v_prefix));
        if (FB_TEXT_FUSE_REDUCE && block_small_path(s, n_q) && gp.n_chunks > 0 && !gp.direct) {
          // the in-block kernel merges the partials: no reduce launch
          rc = validate_prefix(&s, a->q_blk, st->k_prefix, st->v_prefix, &sel, st->a_out,
                               st->l_out, ar, lr);
          if (rc != FB_OK) return rc;
          PrefixHooks hk;
          memset(&hk, 0, sizeof(hk));
          hk.defer = &fused;
          rc = run_prefix(s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, &sel, st->a_out,
                          st->l_out, ar, lr, st->ws, st->ws_bytes, stream, &hk);
          if (rc != FB_OK) return rc;
          has_fused = true;
        } else {
          rc = fb_prefix_attn(&s, a->q_blk, st->k_prefix, st->v_prefix, nullptr, &sel, st->a_out,
                              st->l_out, ar, lr, st->ws, st->ws_bytes, stream);
          if (rc != FB_OK) return rc;
        }
      } else {
        rc = token_step(0, 0);                     // forced reuse: no token active
        if (rc != FB_OK) return rc;
      }
      break;
    }
    default:
      return FB_ERR_INVALID_ARGUMENT;
  }
  rc = block_merge(&s, a->q_blk, a->k_blk, a->v_blk, st->a_out, st->l_out, a->a_full, a->l_full,
                   nullptr, nullptr, has_fused ? &fused : nullptr, st->a_out, st->l_out, q_dst,
                   stream);
  if (rc != FB_OK) return rc;
  st->step += 1;
  return FB_OK;
}

fb_status fb_step_next_block(fb_step_state* st, fb_kv_cache* c, fb_tensor k_blk, fb_tensor v_blk,
                             hipStream_t stream) {
  if (!st || !c) return FB_ERR_INVALID_ARGUMENT;
  fb_status rc = check_shape(&st->shape);
  if (rc != FB_OK) return rc;
  // the state's prefix is the cache's first n_tok tokens
  const fb_tensor& kp = st->k_prefix;
  const fb_tensor& vp = st->v_prefix;
  if (kp.ptr != c->k || vp.ptr != c->v || kp.n_tok != c->n_tok || vp.n_tok != c->n_tok ||
      kp.stride_tok != c->stride_tok || kp.stride_head != c->stride_head ||
      vp.stride_tok != c->stride_tok || vp.stride_head != c->stride_head)
    return FB_ERR_INVALID_ARGUMENT;
  const int64_t n_old = c->n_tok;
  const bool sparse = st->mode == FB_STEP_SPARSE;
  const bool incremental = sparse && st->page_cap > 0 && st->meta_ready;
  if (sparse) {
    if (st->page_size < 1 || st->page_cap < 0) return FB_ERR_INVALID_ARGUMENT;
    if (k_blk.n_tok < 0 || k_blk.n_tok > c->capacity - n_old) return FB_ERR_INVALID_ARGUMENT;
    const int64_t n_pages = (n_old + k_blk.n_tok + st->page_size - 1) / st->page_size;
    if (st->page_cap > 0 && n_pages > st->page_cap) return FB_ERR_INVALID_ARGUMENT;
    if (incremental && (!st->kmin || !st->kmax)) return FB_ERR_INVALID_ARGUMENT;
  }
  rc = fb_kv_append(&st->shape, c, k_blk, v_blk, stream);
  if (rc != FB_OK) return rc;
  st->k_prefix.n_tok = c->n_tok;
  st->v_prefix.n_tok = c->n_tok;
  st->step = 0;
  if (sparse) {
    if (!incremental) {
      st->meta_ready = 0;              // rebuilt at the next refresh step
    } else {
      rc = fb_page_meta_update(&st->shape, st->k_prefix, st->page_size, n_old, st->page_cap,
                               st->kmin, st->kmax, stream);
      if (rc != FB_OK) {
        st->meta_ready = 0;
        return rc;
      }
    }
  }
  return FB_OK;
}

}  // extern "C"
