/*
 * flashblock.h -- C ABI of the MI355X (gfx950) FlashBlock block-diffusion
 * attention step.
 *
 * The method (FlashBlock: Attention Caching for Efficient Long-Context Block
 * Diffusion, technical summary, s2 "core mechanism"): the B queries of the
 * block being denoised attend over two key sets, J_out (every token outside
 * the block: the long, static prefix KV cache) and J_in (the block's own
 * tokens). The block-external output A_out and its log-normaliser
 * L_out = ln Z_out are cached and reused on later denoising steps; only the
 * block-internal pair (A_in, L_in) is recomputed, and the two are combined
 * by the log-space composition
 *     m = max(L_out, L_in)
 *     A_full = (e^{L_out-m} A_out + e^{L_in-m} A_in) / (e^{L_out-m} + e^{L_in-m}).
 * A reuse controller (same page, s2 "adaptive reuse strategies") recomputes
 * the cached pair when the count of updated tokens M reaches tau (text), or
 * per head when the head's similarity is not above gamma (video); unselected
 * keys of a sparse attention can play the role of J_out (sparse
 * compatibility), with the page selection of LoSA (Locality Aware Sparse
 * Attention for Block-Wise Diffusion Language Models, s2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is device memory owned by the caller, unless it
 *    is documented as host memory. The library allocates nothing, keeps no
 *    global state (except the per-device scratch array of
 *    fb_prefix_attn_noalloc) and is reentrant: calls on different streams
 *    may overlap as long as they do not share output buffers (calls of
 *    fb_prefix_attn_noalloc on one GPU may not overlap at all).
 *  - Tensors of q, k, v are described by fb_tensor: element strides between
 *    tokens and between heads; the head dimension is contiguous (stride 1).
 *    Base pointers must be 16-byte aligned and token/head strides multiples
 *    of 8 elements (16 bytes for bf16, 32 for fp32).
 *  - Outputs are fp32, contiguous: A as [n_q, Hq, head_dim], L as [n_q, Hq].
 *  - L is a natural logarithm of the softmax denominator over the *scaled*
 *    scores s_j = scale * q . k_j. An empty key set yields A = 0, L = -inf.
 *  - Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
 *  - Mask bytes: 1 = reuse (skip the recompute), 0 = recompute.
 *  - Every entry point validates its arguments on the host before any
 *    launch and returns a status; none throws or aborts. Launch failures map
 *    to FB_ERR_DEVICE. Faults inside kernels surface, as with any HIP work,
 *    at the caller's next synchronisation.
 *  - All work is enqueued on the given stream with no host synchronisation;
 *    decisions taken on the device (masks, counts) are consumed on the
 *    device.
 */
#ifndef FLASHBLOCK_H
#define FLASHBLOCK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FB_ABI_VERSION 3

typedef enum {
  FB_OK = 0,
  FB_ERR_INVALID_ARGUMENT = 1,   /* bad shape, stride, pointer or value       */
  FB_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. head_dim) */
  FB_ERR_WORKSPACE_TOO_SMALL = 3,
  FB_ERR_DEVICE = 4              /* a HIP launch or runtime call failed       */
} fb_status;

typedef enum { FB_BF16 = 0, FB_F32 = 1 } fb_dtype;

typedef struct {
  int32_t n_q_heads;    /* Hq >= 1                                         */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0                         */
  int32_t head_dim;     /* 64 or 128                                       */
  float scale;          /* softmax scale on q . k (usually 1/sqrt(d)), > 0 */
  fb_dtype dtype;       /* element type of q, k, v                         */
} fb_attn_shape;

typedef struct {
  const void* ptr;      /* device, 16-byte aligned; may be NULL iff n_tok == 0 */
  int64_t n_tok;        /* tokens                                              */
  int64_t stride_tok;   /* elements between consecutive tokens                 */
  int64_t stride_head;  /* elements between consecutive heads                  */
} fb_tensor;

/* ------------------------------------------------------------------------ *
 * Sparse page selection (optional; FlashBlock s2 sparse compatibility,     *
 * LoSA s2 QUEST-selected sparse attention for active tokens).               *
 * ------------------------------------------------------------------------ */
typedef enum {
  FB_SEL_DENSE = 0,   /* every prefix key                                     */
  FB_SEL_SPLIT = 1,   /* one pass: selected pages and their complement        */
  FB_SEL_GATHER = 2   /* selected pages of active rows only, merged with the
                         cached residual                                       */
} fb_sel_mode;

typedef struct {
  fb_sel_mode mode;
  int32_t page_size;      /* tokens per page (16); page p = tokens [p*ps, p*ps+ps) */
  int32_t k_pages;        /* selected pages per (query token, KV head), >= 0     */
  const int32_t* pages;   /* [n_q, Hkv, k_pages] page ids, strictly ascending;
                             ids outside [0, ceil(n_kv / page_size)) select
                             nothing                                           */
  const uint8_t* active;  /* GATHER: [n_q] 1 = the row recomputes; NULL = all    */
  const uint32_t* bitmap; /* NULL, or the same selection as bitmaps, written by
                             fb_page_bitmap: [n_q, Hkv, ceil(n_pages / 32)]
                             uint32, bit p of row (t, g) set iff page p is in
                             S_{t,g}. Given, `pages` is not read and no
                             selection prep runs: a GATHER pass then takes
                             the union over the active rows in its own
                             workgroups (one launch fewer)                    */
} fb_page_sel;

/* ------------------------------------------------------------------------ *
 * fb_prefix_attn -- the block-external pass over J_out.                    *
 * FlashBlock s2 "core mechanism": A_out and L_out = log Z_out over the      *
 * tokens outside the block, computed when the controller asks for it.      *
 *                                                                           *
 * q [n_q, Hq, d]; k, v [n_kv, Hkv, d] (any token/head strides). Head-major *
 *   storage (each KV head's keys contiguous: stride_head >= n_kv *          *
 *   stride_tok) streams fastest; the workspace size does not depend on the  *
 *   layout (the kernel it selects may change results at rounding level).    *
 * head_reuse_mask: NULL, or device [Hq]; heads with byte 1 are skipped and  *
 *   their rows of every output are left untouched.                          *
 * sel: NULL or mode DENSE -> a_out, l_out over all n_kv keys; a_res, l_res  *
 *   must be NULL.                                                            *
 *   SPLIT  -> a_res, l_res (outputs) = the pair over the keys NOT in the    *
 *   row's selected pages; a_out, l_out = the pair over all keys (the merge  *
 *   of the selected part and the residual).                                  *
 *   GATHER -> a_res, l_res are INPUTS (the cached residual); for rows whose  *
 *   active byte is 1, a_out, l_out = merge(pair over the selected pages,     *
 *   cached residual); other rows are left untouched. With a_res and l_res   *
 *   both NULL there is no residual: a_out, l_out = the pair over the         *
 *   selected pages alone (LoSA s2: sparse attention for active tokens).      *
 * ws: device workspace of at least fb_prefix_attn_workspace() bytes (split- *
 *   K partials); may be NULL when that size is 0.                            *
 * Errors: INVALID_ARGUMENT on bad shape/stride/alignment/NULL, n_q < 1,     *
 *   n_kv < 0, k/v token counts that differ; UNSUPPORTED for head_dim not   *
 *   in {64,128}, and for a SPLIT/GATHER selection on the bf16, d = 128,     *
 *   page-size-multiple-of-16 kernel over more than 8,355,840 keys (the      *
 *   split-K reduce merges at most 1024 chunks of 8,160 keys); nothing is    *
 *   launched then. WORKSPACE_TOO_SMALL. Page ids are device data and are    *
 *   not validated (see fb_page_sel).                                         *
 * ------------------------------------------------------------------------ */
size_t fb_prefix_attn_workspace(const fb_attn_shape* shape, int64_t n_q,
                                int64_t n_kv, const fb_page_sel* sel);
fb_status fb_prefix_attn(const fb_attn_shape* shape, fb_tensor q, fb_tensor k,
                         fb_tensor v, const uint8_t* head_reuse_mask,
                         const fb_page_sel* sel, float* a_out, float* l_out,
                         float* a_res, float* l_res, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_prefix_attn_noalloc -- fb_prefix_attn without a workspace argument,    *
 * for callers that cannot allocate device memory (code under HIP graph      *
 * capture, tight serving loops, harnesses that forbid allocation). The      *
 * split-K partials (and a sparse selection's bitmaps and page union) live  *
 * in a fixed 16 MiB device array inside the library, one copy per GPU the  *
 * library runs on, held until the process ends; its address is looked up   *
 * on the first call on each device. Arguments and results as               *
 * fb_prefix_attn. The call allocates nothing (no hipMalloc, no library      *
 * routine that allocates).                                                  *
 * stream: must belong to the current device (NULL: the current device's     *
 *   null stream).                                                           *
 * Every call on one GPU shares that GPU's array: calls that overlap on one  *
 * GPU (on different streams, or from different host threads) race and may  *
 * return wrong results; calls in one stream's order are safe. No byte of    *
 * the array needs to start at any value: a call reads only what it wrote    *
 * earlier in the same call.                                                 *
 * Errors: as fb_prefix_attn, and WORKSPACE_TOO_SMALL when the call needs    *
 *   more than 16 MiB (fb_prefix_attn_workspace() > 16 MiB, e.g. many query  *
 *   rows over a long prefix); INVALID_ARGUMENT for a stream of another      *
 *   device; UNSUPPORTED for device ordinals >= 64. Nothing is launched on  *
 *   an error.                                                               *
 * ------------------------------------------------------------------------ */
#define FB_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
fb_status fb_prefix_attn_noalloc(const fb_attn_shape* shape, fb_tensor q,
                                 fb_tensor k, fb_tensor v,
                                 const uint8_t* head_reuse_mask,
                                 const fb_page_sel* sel, float* a_out,
                                 float* l_out, float* a_res, float* l_res,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_block_attn_merge -- the block-internal pass and the log-space merge.  *
 * FlashBlock s2 "core mechanism": A_in, L_in over J_in (the block's own     *
 * B tokens; every block query sees every block key -- the pages state no    *
 * in-block mask), then A_full = the log-space composition of the cached      *
 * (A_out, L_out) with (A_in, L_in).                                          *
 *                                                                            *
 * q_blk [n_q, Hq, d]; k_blk, v_blk [n_q, Hkv, d]; a_out, l_out: the cached  *
 * pair (inputs); l_out may hold -inf (no cached side: A_full = A_in).       *
 * a_full (required), l_full, a_in, l_in (nullable) outputs.                 *
 * ws: unused (fb_block_attn_merge_workspace() returns 0); may be NULL.      *
 * Errors: as fb_prefix_attn; when a KV head serves >= 128 query rows (bf16, *
 * d = 128: the MFMA pass) a_out, a_full and a_in must be 16-byte aligned;   *
 * UNSUPPORTED for more than 65535 block tokens on the small-block path.    *
 * ------------------------------------------------------------------------ */
size_t fb_block_attn_merge_workspace(const fb_attn_shape* shape, int64_t n_q);
fb_status fb_block_attn_merge(const fb_attn_shape* shape, fb_tensor q_blk,
                              fb_tensor k_blk, fb_tensor v_blk,
                              const float* a_out, const float* l_out,
                              float* a_full, float* l_full, float* a_in,
                              float* l_in, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_reuse_decide -- the reuse controller.                                  *
 * ------------------------------------------------------------------------ */
typedef enum {
  /* FlashBlock s2 threshold reuse: M = #{i : ids_cur[i] != ids_prev[i]};
     mask[h] = (M < tau) for every head, unless force says otherwise.
     ids_prev holds the previous step's ids, or, to count the drift since the
     last recompute (since_refresh = 1), the ids of that step: ids_store then
     receives ids_cur only when the decision is to recompute.                */
  FB_REUSE_COUNT = 0,
  /* FlashBlock s2 per-head selection: sim[h] = cosine of head h's output in
     a_probe vs a_cached, flattened over [n_q, d], float64, clamped to
     [-1, 1] (both all-zero -> 1, one zero -> 0); for heads with
     mask_in[h] == 0: sim[h] updated, mask[h] = (sim[h] > gamma); heads with
     mask_in[h] == 1 keep sim[h] and get mask[h] = 1.                        */
  FB_REUSE_HEAD_COS = 1,
  /* LoSA s2 token classification: mse[t] = (sum over heads, in head order,
     of the head's sum over dims, in dim order, of (q_cur - q_prev)^2) / (Hq*d),
     in float64 without fused multiply-add; cutoff = the ceil(pct/100 * n_q)-th
     smallest mse; active[t] = mse[t] > cutoff.                              */
  FB_REUSE_ACTIVE_MSE = 2
} fb_reuse_mode;

typedef struct {
  fb_reuse_mode mode;
  int32_t n_q;              /* block tokens / queries                         */
  int32_t n_heads;          /* Hq                                             */
  int32_t head_dim;         /* d (HEAD_COS, ACTIVE_MSE)                       */
  /* COUNT */
  const int32_t* ids_prev;  /* [n_q]                                          */
  const int32_t* ids_cur;   /* [n_q]                                          */
  int32_t tau;              /* reuse iff M < tau                              */
  int32_t force;            /* -1 decide; 0 force recompute; 1 force reuse    */
  int32_t* m_count;         /* out [1], nullable                              */
  int32_t* ids_store;       /* nullable out [n_q]: receives ids_cur after the
                               count (may alias ids_prev)                      */
  /* HEAD_COS */
  const float* a_cached;    /* [n_q, Hq, d]                                   */
  const float* a_probe;     /* [n_q, Hq, d]                                   */
  const uint8_t* mask_in;   /* [Hq] nullable (= all zero)                     */
  double gamma;
  double* sim;              /* in/out [Hq]                                    */
  /* ACTIVE_MSE */
  const void* q_prev;       /* [n_q, Hq, d] contiguous, dtype below           */
  const void* q_cur;        /* [n_q, Hq, d] contiguous                        */
  fb_dtype dtype;
  int32_t pct;              /* 1..100                                         */
  double* mse;              /* out [n_q], nullable                            */
  uint8_t* active;          /* out [n_q]                                      */
  /* output of COUNT and HEAD_COS */
  uint8_t* mask;            /* [Hq]                                           */
  void* ws;                 /* device workspace >= fb_reuse_decide_workspace  */
  size_t ws_bytes;
  int32_t since_refresh;    /* COUNT: 1 = ids_store only on recompute         */
} fb_reuse_args;

size_t fb_reuse_decide_workspace(const fb_reuse_args* args);
fb_status fb_reuse_decide(const fb_reuse_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * Page metadata and selection (optional sparse subsystem).                  *
 * fb_page_meta: kmin, kmax [Hkv, P, d] (dtype of k, 16-byte aligned),      *
 *   P = ceil(n_kv / ps):                                                    *
 *   elementwise min / max of the page's keys (the last page may be short).  *
 * fb_page_meta_update: the same metadata kept in storage of page_cap pages  *
 *   per KV head ([Hkv, page_cap, d]) for a cache that grows: given storage  *
 *   that describes the first n_tok_old tokens of k, recomputes the pages     *
 *   that tokens [n_tok_old, k.n_tok) touch -- the old partial last page and  *
 *   the new ones, pages floor(n_tok_old / ps) .. ceil(k.n_tok / ps) - 1 --    *
 *   so the storage then equals fb_page_meta over all k.n_tok tokens. Pages   *
 *   wholly inside the old prefix keep their min / max (it depends on their   *
 *   own tokens only). n_tok_old = 0 builds the whole storage.                *
 *   INVALID_ARGUMENT if n_tok_old > k.n_tok or ceil(k.n_tok / ps) > page_cap.*
 * fb_page_select: bound[t, g, p] = max over the query heads h of group g of *
 *   sum_{j = 0..d-1, in order} max(q[t,h,j]*kmin[g,p,j], q[t,h,j]*kmax[g,p,j])*
 *   in float64 (each product of two bf16 or two fp32 values is exact, so a  *
 *   fused multiply-add rounds as a multiply then an add would);             *
 *   pages[t, g, :] = the k_pages                                            *
 *   pages of largest bound (ties: lower page id first), listed ascending.    *
 *   kmin/kmax (16-byte aligned) hold page_cap pages per KV head (0:         *
 *   n_pages, packed).                                                       *
 *   active (nullable, device [n_q]): tokens whose byte is 0 are skipped;    *
 *   their rows of bound and pages are left untouched.                       *
 *   bound may be NULL (then it lives in ws).                                  *
 *   UNSUPPORTED for more than 65,535 block tokens, or when one token's      *
 *   G * d query values and 64 page rows of d + 1 floats exceed 64 KB (group *
 *   sizes other than 1, 2, 4, 8: e.g. G > 63 at d = 128).                   *
 * ------------------------------------------------------------------------ */
fb_status fb_page_meta(const fb_attn_shape* shape, fb_tensor k,
                       int32_t page_size, void* kmin, void* kmax,
                       hipStream_t stream);
fb_status fb_page_meta_update(const fb_attn_shape* shape, fb_tensor k,
                              int32_t page_size, int64_t n_tok_old,
                              int64_t page_cap, void* kmin, void* kmax,
                              hipStream_t stream);
size_t fb_page_select_workspace(const fb_attn_shape* shape, int64_t n_q,
                                int64_t n_pages);
fb_status fb_page_select(const fb_attn_shape* shape, fb_tensor q,
                         const void* kmin, const void* kmax, int64_t n_pages,
                         int64_t page_cap, int32_t k_pages,
                         const uint8_t* active, int32_t* pages, double* bound,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_page_bitmap -- a page selection as bitmaps (for fb_page_sel.bitmap and *
 * fb_step_state.sel_bitmap): bitmap[(t Hkv + g) ceil(n_pages / 32) + w]     *
 * bit b set iff page 32 w + b is in pages[t][g][0 .. k_pages). LoSA s2 /    *
 * FlashBlock s2 sparse compatibility: the selection a GATHER pass masks     *
 * its rows with, built once per selection instead of once per pass.        *
 * pages [n_q, Hkv, k_pages] device int32 (ids outside [0, n_pages) set no  *
 * bit); bitmap device out.                                                  *
 * Errors: INVALID_ARGUMENT for a bad shape, n_q < 1, n_pages < 1 or beyond *
 *   INT32_MAX, k_pages outside [0, n_pages], NULL pointers (pages when      *
 *   k_pages > 0); UNSUPPORTED when a row exceeds 16,384 words.              *
 * ------------------------------------------------------------------------ */
fb_status fb_page_bitmap(const fb_attn_shape* shape, const int32_t* pages,
                         int64_t n_q, int64_t n_pages, int32_t k_pages,
                         uint32_t* bitmap, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_proxy_decide -- singular-proxy identification (SPA-Cache, "Proxy       *
 * singolari per la caching adattiva nei modelli linguistici diffusivi",     *
 * methodology s1): which tokens to recompute, found from rank-r proxies of  *
 * their value states.                                                       *
 *                                                                           *
 * x [n_tok, d_model] input states (dtype; row stride x_stride elements);    *
 * factor [d_model, rank] contiguous, 16-byte aligned (dtype): U_r         *
 * diag(sigma_r) of the value                                                *
 * projection's truncated SVD; cache [n_tok, rank] float64: the proxy kept   *
 * per token from the step it was last recomputed (in/out).                  *
 *   proxy p[t][i] = sum_c x[t][c] factor[c][i], float64 (products of two  *
 *     bf16 or two fp32 values are exact in float64; the sums round in the   *
 *     library's own order, within a few ulps of sum |x factor|);            *
 *   sim[t] = the cosine of p[t] and cache[t]: dot / sqrt(|p|^2 |c|^2),      *
 *     float64, clamped to [-1, 1]; both norms 0 -> 1, one -> 0 (a proxy    *
 *     equal to its cache scores exactly 1).                                 *
 * init = 1: cache <- p for every token, mask all 1 (sim, selected unused).  *
 * init = 0: selected [n_select] = the n_select tokens of lowest sim (ties:  *
 *   lower id), ascending; mask[t] = 1 for them, 0 otherwise; their cache    *
 *   rows <- p. sim (nullable) receives every token's similarity, proxy    *
 *   (nullable) every current proxy.                                         *
 * Errors: INVALID_ARGUMENT for n_tok < 1, d_model < 1, x_stride < d_model, *
 *   NULL x / factor / cache / mask (selected when n_select > 0), n_select   *
 *   outside [0, n_tok], init not 0 or 1; UNSUPPORTED for rank not a        *
 *   multiple of 32 in [32, 128]; WORKSPACE_TOO_SMALL.                       *
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_tok;           /* N                                                */
  int32_t d_model;         /* D                                                */
  int32_t rank;            /* r                                                */
  fb_dtype dtype;          /* of x and factor                                  */
  const void* x;           /* [n_tok, d_model]                                 */
  int64_t x_stride;        /* elements between tokens                          */
  const void* factor;      /* [d_model, rank]                                  */
  double* cache;           /* [n_tok, rank] in/out                             */
  int32_t n_select;        /* tokens to recompute (init = 0)                   */
  int32_t init;            /* 1: first step, every token recomputed            */
  double* sim;             /* out [n_tok], nullable                            */
  int32_t* selected;       /* out [n_select]                                   */
  uint8_t* mask;           /* out [n_tok]                                      */
  double* proxy;           /* out [n_tok, rank], nullable                      */
  void* ws;                /* device workspace >= fb_proxy_decide_workspace() */
  size_t ws_bytes;
} fb_proxy_args;

size_t fb_proxy_decide_workspace(const fb_proxy_args* args);
fb_status fb_proxy_decide(const fb_proxy_args* args, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_layer_budgets -- per-layer update budgets over depth (SPA-Cache,       *
 * methodology s2 "adaptive budget allocation": middle layers drift most,   *
 * so they recompute more tokens; first and last layers cache more).        *
 * HOST function (no device work, no stream).                                *
 *   g(l) = exp(-(l - mu)^2 / (2 s^2)), s = s_left for l < mu, s_right     *
 *   otherwise; ratio(l) = floor + (peak - floor) g(l) with peak chosen so  *
 *   that the mean ratio over the n_layers layers is mean_ratio;            *
 *   counts[l] = floor(ratio(l) n_tok + 1/2), clamped to [0, n_tok].         *
 * ratios (host [n_layers], nullable), counts (host [n_layers]).             *
 * Errors: INVALID_ARGUMENT for n_layers < 1, n_tok < 0, s_left or s_right  *
 *   <= 0, a non-finite value, or not 0 <= floor <= mean_ratio <= 1.        *
 * ------------------------------------------------------------------------ */
fb_status fb_layer_budgets(int32_t n_layers, int32_t n_tok, double mean_ratio,
                           double floor_ratio, double mu, double s_left,
                           double s_right, double* ratios, int32_t* counts);

/* ------------------------------------------------------------------------ *
 * fb_layer_taus -- per-layer reuse thresholds of a stack of FlashBlock       *
 * layers from per-layer update budgets. HOST function.                      *
 * FlashBlock s2 "adaptive reuse strategies" (a layer reuses its cached      *
 * pair while fewer than tau block tokens changed) under SPA-Cache           *
 * methodology s2 "adaptive budget allocation" (a layer whose states drift   *
 * more gets a larger update budget): a layer's staleness tolerance is       *
 * inversely proportional to its budget, scaled so that a layer at the mean  *
 * budget keeps base_tau:                                                    *
 *   taus[l] = floor(base_tau mean_ratio / ratios[l] + 1/2), clamped to      *
 *   [1, block + 1]; ratios[l] <= 0 -> block + 1 (the layer never            *
 *   recomputes after a block's first step).                                 *
 * ratios (host [n_layers], e.g. from fb_layer_budgets), taus (host out).    *
 * Errors: INVALID_ARGUMENT for n_layers, block or base_tau < 1, NULL        *
 *   arrays, a non-finite ratio, or mean_ratio outside (0, 1].               *
 * ------------------------------------------------------------------------ */
fb_status fb_layer_taus(int32_t n_layers, int32_t block, int32_t base_tau,
                        double mean_ratio, const double* ratios, int32_t* taus);

/* ------------------------------------------------------------------------ *
 * Growing prefix cache (FlashBlock s1 problem statement: block-wise         *
 * decoding attends over a KV cache that grows as blocks finish).            *
 *                                                                           *
 * fb_kv_cache is a host struct owned by the caller describing device        *
 * storage for up to `capacity` tokens of K and V ([capacity, Hkv, d] under  *
 * the strides, token-major or head-major, both tensors alike); the first    *
 * n_tok tokens are the prefix J_out. The prefix as an fb_tensor is          *
 * {k, n_tok, stride_tok, stride_head}.                                       *
 *                                                                           *
 * fb_kv_append: copies k_blk, v_blk [B, Hkv, d] (the finished block, any    *
 *   strides) into tokens [n_tok, n_tok + B) of the storage and, once the    *
 *   copy is enqueued, sets cache->n_tok += B (host). A block already written *
 *   in place (k_blk.ptr at token n_tok of the storage, same strides) is not  *
 *   copied. The block rows must not otherwise overlap the destination.       *
 *   Errors: INVALID_ARGUMENT for bad shape/strides/alignment, NULL storage,  *
 *   k/v token counts that differ, or n_tok + B > capacity.                   *
 * ------------------------------------------------------------------------ */
typedef struct {
  void* k;                 /* device storage                                   */
  void* v;
  int64_t capacity;        /* tokens the storage holds                         */
  int64_t n_tok;           /* tokens in use (0 <= n_tok <= capacity)           */
  int64_t stride_tok;      /* elements between tokens (k and v alike)          */
  int64_t stride_head;     /* elements between heads                           */
} fb_kv_cache;

fb_status fb_kv_append(const fb_attn_shape* shape, fb_kv_cache* cache,
                       fb_tensor k_blk, fb_tensor v_blk, hipStream_t stream);

/* ------------------------------------------------------------------------ *
 * fb_step -- one denoising step of one block, all launches on `stream`.    *
 *                                                                           *
 * TEXT   (FlashBlock s2 threshold reuse): COUNT decision on the device ->  *
 *        prefix pass for the heads that recompute (every head at step 0)   *
 *        into the cache (a_out, l_out) -> in-block pass + merge.            *
 * VIDEO  (FlashBlock s2 per-head selection, probe reading): step 0 fills   *
 *        the cache; at later steps heads with mask 0 recompute into the     *
 *        probe buffer, HEAD_COS compares probe and cache and writes         *
 *        mask_next, the probe replaces the cache for those heads; the       *
 *        in-block pass merges with the cache. mask and mask_next swap.      *
 * SPARSE (FlashBlock s2 sparse compatibility + LoSA s2 workflow): step 0   *
 *        builds page metadata (once per prefix), selects pages, runs the    *
 *        SPLIT pass (cache + residual); later steps classify tokens by      *
 *        query MSE and run the GATHER pass for active rows. With            *
 *        sparse_reselect = 1 (LoSA s2 workflow as it stands): step 0 is a    *
 *        dense pass; later steps select pages with the step's queries for   *
 *        the active tokens (pages rows of the others are left as they were) *
 *        and run GATHER for them with no residual (a_res, l_res unused).    *
 *        Blocks with                                                        *
 *        n_q > 1024 or n_q * Hq > 4096 need a contiguous q_blk              *
 *        (UNSUPPORTED otherwise).                                           *
 *                                                                           *
 * fb_step_state is a host struct owned by the caller; `step` counts the    *
 * steps of the current block (set it to 0 at a new block). Buffers it       *
 * points to are caller-owned device memory sized as documented per field.  *
 *                                                                           *
 * fb_step_next_block -- the outer loop (FlashBlock s1: the cache grows by   *
 * each finished block). Appends the finished block's k_blk, v_blk to the    *
 * prefix storage `cache` (fb_kv_append), sets k_prefix / v_prefix to the    *
 * grown prefix, brings SPARSE page metadata up to date incrementally        *
 * when page_cap > 0 (fb_page_meta_update; INVALID_ARGUMENT if the new page  *
 * count exceeds page_cap) -- with page_cap = 0 the packed metadata is       *
 * rebuilt at the next refresh step, into kmin / kmax that must then hold    *
 * the new page count -- and sets step = 0, so the next fb_step starts the   *
 * next block with a full compute. k_prefix and                              *
 * v_prefix must view the first cache->n_tok tokens of cache->k, cache->v    *
 * (same pointers and strides). The workspace the next block needs may grow  *
 * with the prefix: query fb_step_workspace() again (fb_step returns         *
 * WORKSPACE_TOO_SMALL otherwise). Errors: INVALID_ARGUMENT when the state   *
 * does not view the cache, or as fb_kv_append; the state is unchanged then. *
 * ------------------------------------------------------------------------ */
typedef enum { FB_STEP_TEXT = 0, FB_STEP_VIDEO = 1, FB_STEP_SPARSE = 2 } fb_step_mode;

typedef struct {
  fb_attn_shape shape;
  fb_step_mode mode;
  int32_t n_q;             /* block queries per step                           */
  fb_tensor k_prefix;      /* J_out keys   [n_kv, Hkv, d]                      */
  fb_tensor v_prefix;      /* J_out values [n_kv, Hkv, d]                      */
  int32_t tau;             /* TEXT                                             */
  double gamma;            /* VIDEO                                            */
  int32_t page_size;       /* SPARSE                                           */
  int32_t k_pages;         /* SPARSE                                           */
  int32_t pct;             /* SPARSE active cutoff percentile                  */
  float* a_out;            /* cache [n_q, Hq, d]                               */
  float* l_out;            /* cache [n_q, Hq]                                  */
  float* a_probe;          /* VIDEO [n_q, Hq, d]                               */
  float* l_probe;          /* VIDEO [n_q, Hq]                                  */
  float* a_res;            /* SPARSE residual [n_q, Hq, d]                     */
  float* l_res;            /* SPARSE residual [n_q, Hq]                        */
  int32_t* ids_prev;       /* TEXT [n_q]                                       */
  int32_t* m_count;        /* TEXT [1]                                         */
  uint8_t* mask;           /* [Hq] reuse flags used by this step               */
  uint8_t* mask_next;      /* VIDEO [Hq]                                       */
  double* sim;             /* VIDEO [Hq]                                       */
  int32_t* pages;          /* SPARSE [n_q, Hkv, k_pages]                       */
  void* kmin;              /* SPARSE [Hkv, page_cap or P, d] (dtype)           */
  void* kmax;              /* SPARSE [Hkv, page_cap or P, d]                   */
  void* q_prev;            /* SPARSE [n_q, Hq, d] contiguous (dtype), 16-B al. */
  double* mse;             /* SPARSE [n_q]                                     */
  uint8_t* active;         /* SPARSE [n_q]                                     */
  void* ws;                /* device workspace >= fb_step_workspace()          */
  size_t ws_bytes;
  int64_t step;            /* host counter; fb_step increments it              */
  int32_t meta_ready;      /* SPARSE: host flag, page metadata built           */
  int64_t page_cap;        /* SPARSE: pages per KV head in kmin / kmax storage;
                              0 = P = ceil(n_kv / page_size) (packed)          */
  int32_t count_since_refresh; /* TEXT: 1 = M counts ids changed since the last
                              recompute step instead of the previous step      */
  int32_t sparse_reselect; /* SPARSE: 1 = LoSA per step (dense first step, pages
                              re-selected each step, no residual)              */
  uint32_t* sel_bitmap;    /* SPARSE, nullable: [n_q, Hkv, ceil(page_cap or P
                              / 32)] uint32. Residual mode: the refresh step
                              writes its selection there as bitmaps; later
                              steps read them instead of rebuilding them, and
                              classify the tokens inside the GATHER pass (two
                              launches a step). sparse_reselect: each step's
                              top-k writes the active tokens' fresh selection
                              there (P <= 8192) and the GATHER pass takes
                              their union itself (no selection prep). Inside
                              the GATHER pass: blocks of up to 64 tokens and
                              unions of up to 1,024 words; beyond, the union
                              (and the classification) take launches of
                              their own (results unchanged)                   */
} fb_step_state;

typedef struct {
  fb_tensor q_blk;         /* [n_q, Hq, d]                                     */
  fb_tensor k_blk;         /* [n_q, Hkv, d]                                    */
  fb_tensor v_blk;         /* [n_q, Hkv, d]                                    */
  const int32_t* ids_cur;  /* TEXT [n_q] token ids of the block at this step   */
  int32_t decision;        /* -1: the device decides; 0: force recompute;
                              1: force reuse (TEXT/VIDEO: no prefix launch)     */
  float* a_full;           /* out [n_q, Hq, d]                                 */
  float* l_full;           /* out [n_q, Hq], nullable                          */
} fb_step_args;

size_t fb_step_workspace(const fb_step_state* st);
fb_status fb_step(fb_step_state* st, const fb_step_args* args,
                  hipStream_t stream);
fb_status fb_step_next_block(fb_step_state* st, fb_kv_cache* cache,
                             fb_tensor k_blk, fb_tensor v_blk,
                             hipStream_t stream);

const char* fb_status_string(fb_status s);
int fb_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASHBLOCK_H */
