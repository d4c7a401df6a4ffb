// fb_internal.h -- types and launchers shared by the library's own sources
// (host ABI layer and the gfx950 kernels). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flashblock.h"

namespace fb {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// The lo part of a bf16 hi + lo split of eight fp32 weights w: bf16(w - hi).
// hi's fp32 values come from its packed pairs themselves (one shift or mask
// each) rather than from a second conversion.
__device__ __forceinline__ bf16x8 bf16_lo_part(f32x8 w, bf16x8 hi) {
  const u32x4v hb = __builtin_bit_cast(u32x4v, hi);
  u32x4v lb;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float h0 = __uint_as_float(hb[c] << 16), h1 = __uint_as_float(hb[c] & 0xffff0000u);
    lb[c] = __builtin_bit_cast(uint32_t,
                               __builtin_convertvector((f32x2){w[2 * c] - h0, w[2 * c + 1] - h1}, bf16x2));
  }
  return __builtin_bit_cast(bf16x8, lb);
}

// Sum over j = 0..d-1, in order, of (cur[j] - prev[j])^2 in float64
// (difference, square, add: no contraction), for bf16 (T = uint16_t bits) or
// fp32 rows; d a multiple of 64, both rows 16-byte aligned. Each 64-dim
// round issues all of its 16-byte loads before the arithmetic, so a row
// costs d / 64 memory round trips.
template <typename T>
__device__ __forceinline__ double sq_diff_sum(const T* prev, const T* cur, int d) {
#pragma clang fp contract(off)
  constexpr int kV = 16 / sizeof(T);               // elements per 16-byte vector
  constexpr int kN = 64 / kV;                      // vectors per 64 dims
  double acc = 0.0;
  for (int j0 = 0; j0 < d; j0 += 64) {
    u32x4v va[kN], vb[kN];
#pragma unroll
    for (int u = 0; u < kN; ++u) {
      va[u] = *reinterpret_cast<const u32x4v*>(prev + j0 + u * kV);
      vb[u] = *reinterpret_cast<const u32x4v*>(cur + j0 + u * kV);
    }
#pragma unroll
    for (int u = 0; u < kN; ++u) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (sizeof(T) == 2) {            // elements 2w (low half), 2w + 1
          const double d0 = static_cast<double>(__uint_as_float(vb[u][w] << 16)) -
                            static_cast<double>(__uint_as_float(va[u][w] << 16));
          const double s0 = d0 * d0;
          acc = acc + s0;
          const double d1 = static_cast<double>(__uint_as_float(vb[u][w] & 0xffff0000u)) -
                            static_cast<double>(__uint_as_float(va[u][w] & 0xffff0000u));
          const double s1 = d1 * d1;
          acc = acc + s1;
        } else {
          const double d0 = static_cast<double>(__uint_as_float(vb[u][w])) -
                            static_cast<double>(__uint_as_float(va[u][w]));
          const double s0 = d0 * d0;
          acc = acc + s0;
        }
      }
    }
  }
  return acc;
}

// Sum over j = 0..31, in order, of (cur[j] - prev[j])^2 in float64
// (difference, square, add: no contraction); both rows 16-byte aligned. All
// loads are issued before the arithmetic.
template <typename T>
__device__ __forceinline__ double sq_diff_sum32(const T* prev, const T* cur) {
#pragma clang fp contract(off)
  constexpr int kV = 16 / sizeof(T);               // elements per 16-byte vector
  constexpr int kN = 32 / kV;
  u32x4v va[kN], vb[kN];
#pragma unroll
  for (int u = 0; u < kN; ++u) {
    va[u] = *reinterpret_cast<const u32x4v*>(prev + u * kV);
    vb[u] = *reinterpret_cast<const u32x4v*>(cur + u * kV);
  }
  double acc = 0.0;
#pragma unroll
  for (int u = 0; u < kN; ++u) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
        const double d0 = static_cast<double>(__uint_as_float(vb[u][w] << 16)) -
                          static_cast<double>(__uint_as_float(va[u][w] << 16));
        const double s0 = d0 * d0;
        acc = acc + s0;
        const double d1 = static_cast<double>(__uint_as_float(vb[u][w] & 0xffff0000u)) -
                          static_cast<double>(__uint_as_float(va[u][w] & 0xffff0000u));
        const double s1 = d1 * d1;
        acc = acc + s1;
      } else {
        const double d0 = static_cast<double>(__uint_as_float(vb[u][w])) -
                          static_cast<double>(__uint_as_float(va[u][w]));
        const double s0 = d0 * d0;
        acc = acc + s0;
      }
    }
  }
  return acc;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A sparse GATHER step's token classification done inside the selection
// prep or the GATHER pass itself: query MSE against q_prev, nearest-rank
// cutoff, active flags (the same arithmetic as the active-step kernel).
struct ActiveFromMse {
  const void* q_prev;           // [n_q, hq, d] contiguous
  const void* q_cur; int64_t q_st, q_sh;
  fb_dtype dt;
  int hq, d, pct;
  double* mse;                  // out [n_q], nullable (written by workgroup 0)
  uint8_t* active;              // out [n_q] (written by workgroup 0)
};

// Where a prefix pass writes its per-row result: either the final outputs
// (chunk_stride 0, one chunk) or split-K partials (chunk-major).
struct RowOut {
  float* a;            // [n_chunks][n_q * Hq][D]  (A normalised)
  float* l;            // [n_chunks][n_q * Hq]     (natural-log normaliser)
  int64_t chunk_stride_rows;  // rows between chunks (n_q * Hq), 0 if final
};

// The text controller's decision taken inside the prefix pass (FlashBlock
// technical summary, s2 "adaptive reuse strategies": reuse while fewer than
// tau of the block's tokens changed). Every wave of every workgroup counts
// the tokens whose id differs from the reference ids (a ballot per 64
// tokens), so all of them take the same decision with no communication; on
// reuse the workgroup exits before any K/V read. The writer (one wave of one
// workgroup) publishes the decision as the head mask and the count. Nothing
// in the pass writes the ids, so every wave reads the same ones.
struct TextDecide {
  const int32_t* ids_ref;       // [n] null: first step of a block (every token counts)
  const int32_t* ids_cur;       // [n]
  int n, tau, force;            // force: -1 the count decides, 0 recompute, 1 reuse
  int hq;
  uint8_t* mask;                // [hq] out: 1 = reuse
  int32_t* m_count;             // out, nullable
};

__device__ __forceinline__ bool text_step_reuse(const TextDecide& d, bool writer) {
  const int lane = threadIdx.x & 63;
  int m = d.n;
  if (d.ids_ref) {
    m = 0;
    for (int i0 = 0; i0 < d.n; i0 += 64) {
      const int i = i0 + lane;
      const bool diff = i < d.n && d.ids_ref[i] != d.ids_cur[i];
      m += __popcll(__ballot(diff));
    }
  }
  const bool reuse = d.force == 1 ? true : (d.force == 0 ? false : m < d.tau);
  if (writer) {
    for (int h = lane; h < d.hq; h += 64) d.mask[h] = reuse ? 1 : 0;
    if (lane == 0 && d.m_count) *d.m_count = m;
  }
  return reuse;
}

struct PrefixParams {
  const void* q; int64_t q_st, q_sh;
  const void* k; const void* v; int64_t kv_st, kv_sh;
  int64_t n_kv;
  int n_q, hq, hkv, group;      // group = Hq / Hkv
  float scale_log2;             // scale * log2(e)
  const uint8_t* mask;          // [Hq] nullable, 1 = skip
  int64_t tiles_per_chunk;      // in units of the kernel's tile
  int n_chunks;
  int n_slabs;                  // MFMA path: row slabs per (chunk, KV head)
  int heads_inner;              // MFMA path: consecutive items = the KV heads of one chunk
  RowOut out;
  // sparse modes
  int sel_mode;                 // FB_SEL_*
  int page_size, k_pages;
  const int32_t* pages;         // [n_q, Hkv, k_pages]
  const uint8_t* active;        // [n_q] nullable
  RowOut out_res;               // SPLIT: residual partials
  // sparse MFMA path
  const uint32_t* bitmap;       // [n_q, Hkv, words] selection bits per (t, g)
  int words;                    // ceil(n_pages / 32)
  int64_t n_pages;
  const int32_t* ulist;         // GATHER: [Hkv, n_pages] union pages, ascending
  const int32_t* ucnt;          // GATHER: [Hkv] union sizes
  // GATHER with caller-built bitmaps: each workgroup derives the union (and
  // its slice of it) from the bitmaps and the active flags itself
  int union_from_bitmap;
  // ... and, with classify, the active flags too (query MSE against q_prev,
  // nearest-rank cutoff; workgroup 0 writes mse / active out)
  int classify;
  ActiveFromMse am;
  // dense text step: the pass decides reuse itself (mask must be null)
  int decide_on;
  TextDecide decide;
};

// Split-K of the many-rows pass sized on the device: when a head mask leaves
// n_on KV groups to compute, the pass takes as many key chunks as keep about
// `target` workgroups busy (at most c_max, every chunk non-empty). The pass
// and the reduce that merges its partials both derive the split from the
// same mask with this function.
struct RowsDyn {
  int on;                       // 1: chunks from the mask (partials + reduce)
  int n_rtiles, hkv, group, c_max, target;
  int64_t n_tiles;              // 32-key tiles of the prefix
};
struct RowsSplit {
  int chunks;
  int64_t tiles_per_chunk;
};
__host__ __device__ inline RowsSplit rows_dyn_split(int n_on, const RowsDyn& d) {
  const int64_t base = static_cast<int64_t>(n_on > 0 ? n_on : 1) * d.n_rtiles;
  int64_t c = (d.target + base / 2) / base;
  if (c < 1) c = 1;
  if (c > d.c_max) c = d.c_max;
  if (c > d.n_tiles) c = d.n_tiles;
  if (c < 1) c = 1;
  const int64_t tpc = (d.n_tiles + c - 1) / c;
  RowsSplit r;
  r.chunks = static_cast<int>((d.n_tiles + tpc - 1) / tpc);
  r.tiles_per_chunk = tpc;
  return r;
}
// KV groups with at least one head the mask does not skip
__host__ __device__ inline int groups_on(const uint8_t* mask, int hkv, int group) {
  if (!mask) return hkv;
  int n = 0;
  for (int g = 0; g < hkv; ++g) {
    bool on = false;
    for (int j = 0; j < group; ++j) on = on || mask[g * group + j] == 0;
    n += on ? 1 : 0;
  }
  return n;
}

struct ReduceParams {
  const float* part_a; const float* part_l;   // [n_chunks][rows][D], [n_chunks][rows]
  const float* part_ra; const float* part_rl; // SPLIT residual partials (nullable)
  int n_chunks;
  int64_t rows;                 // n_q * Hq
  int hq, d;
  const uint8_t* mask;          // [Hq] nullable
  const uint8_t* active;        // [n_q] nullable (GATHER)
  const float* res_a; const float* res_l;     // GATHER: cached residual input
  float* a_out; float* l_out;   // merged (all partials [+ residual])
  float* a_res; float* l_res;   // SPLIT: residual-only merge
  RowsDyn dyn;                  // dyn.on: n_chunks = the many-rows pass's split from the mask
  // optional: every row (t, h) copies its query q_src[t][h][:] (d elements of
  // q_esize bytes, strides in elements) to q_dst[(t * hq + h) * d], before
  // anything else (a sparse step's q_prev <- q_cur, after every read of it)
  const void* q_src; int64_t q_st, q_sh; void* q_dst; int q_esize;
};


// ---- launchers (return hipError_t of the launch) -----------------------
// prefix pass
int prefix_tile_tokens(int path);               // tokens per tile of a path
hipError_t launch_prefix_generic(const PrefixParams& p, fb_dtype dt, int d, hipStream_t s);
hipError_t launch_prefix_mfma(const PrefixParams& p, int row_blocks, hipStream_t s);
int prefix_mfma_occupancy(int row_blocks);      // workgroups per CU of that kernel
hipError_t launch_prefix_reduce(const ReduceParams& p, hipStream_t s);
// sparse MFMA path (bf16, d = 128, page size a multiple of 16)
hipError_t launch_sel_bitmap(const int32_t* pages, int n_rows, int k_pages, int words, int n_pages,
                             uint32_t* bitmap, hipStream_t s);
hipError_t launch_sel_union(const uint32_t* bitmap, const uint8_t* active, int n_q, int hkv,
                            int words, int32_t* ulist, int32_t* ucnt, int n_pages, hipStream_t s);
bool sel_prep_fits(int n_q, int words);         // bitmaps of one KV group fit in LDS
bool gather_union_fits(int n_q, int words);     // GATHER derives the union from bitmaps itself
bool gather_classify_fits(int n_q, int hq);     // ... and classifies the tokens itself
hipError_t launch_sel_prep(const int32_t* pages, int n_q, int hkv, int k_pages, int words,
                           int n_pages, const uint8_t* active, int do_union, uint32_t* bitmap,
                           int32_t* ulist, int32_t* ucnt, hipStream_t s);
bool sel_prep_mse_fits(int n_q, int hq, int words);
hipError_t launch_sel_prep_mse(const int32_t* pages, int n_q, int hkv, int k_pages, int words,
                               int n_pages, const ActiveFromMse& am, uint32_t* bitmap,
                               int32_t* ulist, int32_t* ucnt, hipStream_t s);
hipError_t launch_prefix_sparse(const PrefixParams& p, hipStream_t s);
int sparse_max_tiles_per_chunk();               // 32-key tiles a GATHER chunk may span
hipError_t launch_prefix_empty(float* a_out, float* l_out, int n_q, int hq, int d,
                               const uint8_t* mask, hipStream_t s);

// in-block pass + merge
struct BlockParams {
  const void* q; int64_t q_st, q_sh;
  const void* k; const void* v; int64_t k_st, k_sh, v_st, v_sh;
  int n_q, hq, hkv, group, d;
  float scale_log2;
  const float* a_out; const float* l_out;
  float* a_full; float* l_full; float* a_in; float* l_in;
  // optional (part_l != NULL): the split-K merge of a dense prefix pass done
  // here instead of in its own reduce launch. Rows of heads with mask[h] = 0
  // (or no mask) merge their n_chunks partials (chunk stride rows), use the
  // result as the cached pair and store it to cache_a / cache_l; rows of
  // heads with mask[h] = 1 read the cached pair as usual.
  const float* part_a; const float* part_l; int n_chunks; int64_t rows;
  const uint8_t* mask; float* cache_a; float* cache_l;
  // ... of a sparse GATHER pass: only rows of tokens with active[t] = 1 merge
  // (the others keep the cached pair), with the cached residual (res_a,
  // res_l; nullable) as one more weighted term
  const uint8_t* active; const float* res_a; const float* res_l;
  void* q_dst;                  // nullable: every row also stores its query to q_dst[t][h][:]
  // nullable: the text step's reference ids, updated after a pass that took
  // the decision itself: ids_store := ids_cur unless ids_keep_on_reuse and
  // the step reused (mask[0] = 1); done by workgroup (0, 0)
  const int32_t* ids_cur; int32_t* ids_store; int ids_n; int ids_keep_on_reuse;
  // a step with no prefix pass (host-forced reuse): workgroup (0, 0) also
  // counts M and publishes the decision first (same wave, each id read
  // before it is overwritten)
  int decide_on;
  TextDecide decide;
};
hipError_t launch_block_small(const BlockParams& p, fb_dtype dt, hipStream_t s);

// many query rows per KV head (prefill regime, bf16, d = 128): either pass
struct RowsParams {
  const void* q; int64_t q_st, q_sh;
  const void* k; const void* v; int64_t k_st, k_sh, v_st, v_sh;
  int64_t n_kv;                 // >= 1
  int n_q, hq, hkv, group;
  float scale_log2;             // scale * log2(e)
  const uint8_t* mask;          // [Hq] nullable, 1 = skip (rows of that head not written)
  int n_rtiles;                 // row tiles per (KV head, chunk)
  int64_t tiles_per_chunk;      // 32-key tiles per chunk
  int n_chunks;
  int n_items;                  // hkv * n_chunks * n_rtiles
  RowOut out;                   // plain: A, L (direct or partials); merge: A_full, L_full
  RowsDyn dyn;                  // dyn.on: split from the mask, n_chunks = its maximum
  const float* a_prev; const float* l_prev;   // merge epilogue: cached pair (null = plain)
  float* a_raw; float* l_raw;   // merge epilogue: optional fresh (A_in, L_in)
};
int rows_tile_rows();           // query rows per workgroup
int rows_occupancy();           // workgroups per CU the kernel is built for
hipError_t launch_rows(const RowsParams& p, hipStream_t s);

// decisions
// ids_store receives ids_cur (on recompute decisions only when store_on_recompute)
hipError_t launch_count(const int32_t* ids_prev, const int32_t* ids_cur, int n_q,
                        int tau, int force, int hq, uint8_t* mask, int32_t* m_count,
                        int32_t* ids_store, int store_on_recompute, hipStream_t s);
// a_copy, l_src, l_copy (nullable): the probe pair is also copied into the
// cache for the heads mask_in leaves (read before it is overwritten)
hipError_t launch_head_cos(const float* a_cached, const float* a_probe, int n_q, int hq,
                           int d, const uint8_t* mask_in, double gamma, double* sim,
                           uint8_t* mask, double* ws, int n_chunks, float* a_copy,
                           const float* l_src, float* l_copy, hipStream_t s);
int head_cos_chunks(int n_q);
hipError_t launch_active_mse(const void* q_prev, const void* q_cur, fb_dtype dt, int n_q,
                             int hq, int d, int pct, double* mse, uint8_t* active,
                             double* ws, hipStream_t s);
// sparse step: active set (mode 1) or active = fill (mode 0), then q_prev <- q_cur
bool active_step_fits(int n_q, int hq);
hipError_t launch_active_step(void* q_prev, const void* q_cur, int64_t q_st, int64_t q_sh,
                              fb_dtype dt, int n_q, int hq, int d, int mode, uint8_t fill, int pct,
                              double* mse, uint8_t* active, hipStream_t s);

// pages
// metadata of pages [p_begin, p_end) of the first n_kv tokens; storage holds
// page_cap pages per KV head ([Hkv][page_cap][d])
hipError_t launch_page_meta(const void* k, int64_t kv_st, int64_t kv_sh, int64_t n_kv,
                            int hkv, int d, int page_size, fb_dtype dt, void* kmin,
                            void* kmax, int64_t p_begin, int64_t p_end, int64_t page_cap,
                            hipStream_t s);
hipError_t launch_page_select(const void* q, int64_t q_st, int64_t q_sh, const void* kmin,
                              const void* kmax, int n_q, int hq, int hkv, int d,
                              int64_t n_pages, int64_t page_cap, int k_pages, fb_dtype dt,
                              const uint8_t* active, double* bound, int32_t* pages,
                              uint32_t* bitmap, hipStream_t s);
// exact top-k of each row of keys [n_rows * hkv][n] (largest first, ties to
// the lower index), the chosen indices listed ascending in out [.., k];
// row_active (nullable, [n_rows]): rows r * hkv + . with byte 0 are skipped;
// flags (nullable, [rows][n]): 1 for the chosen indices, 0 for the others;
// bitmap (nullable, [rows][ceil(n / 32)], n <= topk_bitmap_max()): the
// chosen indices as bits (rows skipped by row_active are not written)
int topk_bitmap_max();
int page_bound_tokens(int n_q, int G, int d);   // tokens per workgroup of the generic bound kernel
hipError_t launch_topk_rows(const double* keys, int n_rows, int hkv, int64_t n, int k,
                            const uint8_t* row_active, int32_t* out, uint8_t* flags,
                            uint32_t* bitmap, hipStream_t s);
// singular-proxy identification: block partials of the proxies, then the
// proxies, cache fill (init) or ranking keys (+ negated keys for the top-k)
bool proxy_rank_ok(int rank);
hipError_t launch_proxy_partials(const void* x, int64_t x_st, const void* factor, fb_dtype dt,
                                 int n_tok, int d_model, int rank, double* part, hipStream_t s);
int proxy_n_blocks(int d_model);
hipError_t launch_proxy_keys(const double* part, int n_blocks, int n_tok, int rank, int init,
                             double* cache, double* proxy, double* sim, double* neg_key,
                             uint8_t* mask, hipStream_t s);
int proxy_select_max_tok();
hipError_t launch_proxy_select(const double* neg_key, int n_tok, int n_select,
                               const double* proxy, int rank, double* cache, uint8_t* mask,
                               uint64_t* words, int32_t* selected, hipStream_t s);
hipError_t launch_proxy_scatter(const int32_t* selected, int n_select, int n_tok,
                                const double* proxy, int rank, double* cache, hipStream_t s);
// the finished block's K/V rows into cache tokens [tok0, tok0 + n_blk); byte
// strides; rows are (d * elem_bytes) bytes, a multiple of 16
hipError_t launch_kv_append(const void* k_src, int64_t ks_t, int64_t ks_h, const void* v_src,
                            int64_t vs_t, int64_t vs_h, void* k_dst, void* v_dst, int64_t d_t,
                            int64_t d_h, int64_t tok0, int n_blk, int hkv, int row_bytes,
                            hipStream_t s);

}  // namespace fb
