// k6_sparse.hip -- the block-external pass with a per-row page selection on
// MFMA (bf16, d = 128, page size a multiple of 16): the sparse subsystem
// FlashBlock pairs with its cache (technical summary, s2 "sparse
// compatibility"), with QUEST-selected pages as in LoSA (s2).
//
// Every row (query token t, query head h of KV group g) has a set S_{t,g} of
// selected pages (shared by the query heads of the group), given as ascending
// page lists; they are turned into one bitmap per (t, g) here.
//   SPLIT  (refresh step): one pass over the whole prefix keeps two online
//          softmax states per row, the selected keys and the rest (the
//          residual), each with its own running max.
//   GATHER (later steps): only the union over the active tokens of their
//          selected pages is read (compacted per KV group, ascending), and
//          each row keeps the keys of its own pages; rows of inactive tokens
//          are not computed. The cached residual is merged by the reduce.
// Both write split-K partials (normalised A, natural-log L) that the
// fixed-order reduce combines.
//
// Workgroup = 4 waves = (chunk of tiles, KV group g, slab of 32 rows); each
// wave streams its own 32-key tiles (w, w+4, ...) through a wave-private LDS
// tile, as two 16-key halves that may come from different pages (GATHER),
// and the four states are merged through LDS at the end. Scores and P.V use
// v_mfma_f32_32x32x16_bf16 exactly as the dense decode kernel does (S^T =
// K.Q^T with lane = row; O^T += V^T.P^T with P as bf16 hi + lo parts).
#include "fb_internal.h"

#include <math.h>

namespace fb {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
#ifndef FB_SPARSE_PREFETCH
#define FB_SPARSE_PREFETCH 1      // GATHER: tiles each wave keeps in flight (1; 2 measured no faster)
#endif
#ifndef FB_SPARSE_GATHER_WAVES
#define FB_SPARSE_GATHER_WAVES 4  // waves of a GATHER workgroup (SPLIT: 4, two softmax states)
#endif
constexpr int kSplitWaves = 4;
constexpr int kGatherWaves = FB_SPARSE_GATHER_WAVES;
constexpr int kTile = 32;
constexpr int kD = 128;
constexpr int kKRow = 272;                   // 17 x 16 B: 16 rows, 16 bank groups
constexpr int kVRow = 320;                   // 20 x 16 B: 4 rows, 4 x 64 B bank spans
constexpr int kKBytes = kTile * kKRow;
constexpr int kVBytes = kTile * kVRow;
constexpr int kWaveLds = kKBytes + kVBytes;
constexpr int kMergeStride = kD + 1;
constexpr float kRescaleLog2 = 8.f;
constexpr int kMaxSlicePages = 512;          // union pages one GATHER chunk may span

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x4 ds_read_tr(const char* lds_generic) {
  auto p = (const __attribute__((address_space(3))) char*)(lds_generic);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// ---------------------------------------------------------------------------
// Selection bitmaps: bit p of row (t, g) set iff page p is in S_{t,g}.
// One workgroup per (t, g); the row is built in LDS (words = ceil(P / 32)).
// ---------------------------------------------------------------------------
// Page ids outside [0, n_pages) select nothing.
__global__ __launch_bounds__(256) void sel_bitmap_kernel(const int32_t* pages, int k_pages,
                                                         int words, int n_pages, uint32_t* bitmap) {
  extern __shared__ uint32_t wl[];
  const int64_t row = blockIdx.x;                  // t * Hkv + g
  for (int i = threadIdx.x; i < words; i += 256) wl[i] = 0u;
  __syncthreads();
  const int32_t* pl = pages + row * k_pages;
  for (int i = threadIdx.x; i < k_pages; i += 256) {
    const uint32_t pg = static_cast<uint32_t>(pl[i]);
    if (pg < static_cast<uint32_t>(n_pages)) atomicOr(&wl[pg >> 5], 1u << (pg & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < words; i += 256) bitmap[row * words + i] = wl[i];
}

// Inclusive prefix sum of c over threads 0..255 of the workgroup, by wave
// shuffles and one exchange of the four wave totals in wsum (exact integer
// sums); total = the sum over those threads. Every thread of the workgroup
// calls it (threads from 256 on pass c = 0 and ignore the result); it holds
// two barriers, the second before wsum can be written again.
__device__ __forceinline__ int scan256(int c, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63 && wave < 4) wsum[wave] = x;
  __syncthreads();
  int pre = 0;
#pragma unroll
  for (int w = 0; w < 3; ++w) pre += w < wave ? wsum[w] : 0;
  total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return x + pre;
}

// Union over the active tokens of their selected pages, per KV group g, as an
// ascending page list and its length. One workgroup per g.
__global__ __launch_bounds__(256) void sel_union_kernel(const uint32_t* bitmap, const uint8_t* active,
                                                        int n_q, int hkv, int words,
                                                        int32_t* ulist, int32_t* ucnt, int n_pages) {
  __shared__ int scan[4];                          // wave totals of scan256
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += 256) {
    const int w = w0 + tid;
    uint32_t u = 0u;
    if (w < words)
      for (int t = 0; t < n_q; ++t)
        if (!active || active[t]) u |= bitmap[(static_cast<int64_t>(t) * hkv + g) * words + w];
    const int c = __popc(u);
    int total;
    int pos = base + scan256(c, scan, total) - c;
    while (u) {
      const int b = __builtin_ctz(u);
      ulist[static_cast<int64_t>(g) * n_pages + pos++] = w * 32 + b;
      u &= u - 1;
    }
    base += total;
  }
  if (tid == 0) ucnt[g] = base;
}

template <typename T> __device__ __forceinline__ double ldd(const T* p);
template <> __device__ __forceinline__ double ldd<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ double ldd<uint16_t>(const uint16_t* p) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*p) << 16));
}

// The selection prep of a sparse GATHER step with the step's token
// classification folded in: every workgroup (one per KV group g) computes
// the query MSE of every token against q_prev -- per (token, head) a float64
// sum over d in order of (cur - prev)^2 (difference, square, add), the
// heads' sums added in order, divided by Hq d -- the nearest-rank cutoff and
// the active flags (MSE strictly above it), exactly as the active-step
// kernel does; workgroup 0 writes them out. Then the bitmaps of group g and
// their union over the active tokens, as in sel_prep_kernel. (q_prev is
// only read here; the caller overwrites it later in the step.)
template <typename T>
__global__ __launch_bounds__(1024) void sel_prep_mse_kernel(const int32_t* pages, int n_q, int hkv,
                                                           int k_pages, int words, int n_pages,
                                                           ActiveFromMse am, uint32_t* bitmap,
                                                           int32_t* ulist, int32_t* ucnt) {
#pragma clang fp contract(off)
  extern __shared__ uint32_t bm[];                 // [n_q][words], then the float64 sums
  __shared__ int scan[4];                          // wave totals of scan256
  __shared__ double cutoff_s;
  __shared__ uint8_t act_s[1024];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int hq = am.hq;
  constexpr int d = 128;                           // the sparse kernels' head_dim
  double* part = reinterpret_cast<double*>(bm + ((n_q * words + 1) & ~1));   // [n_q * hq]
  double* mse_s = part + n_q * hq;                                            // [n_q]
  const T* qp = static_cast<const T*>(am.q_prev);
  const T* qc = static_cast<const T*>(am.q_cur);
  const int chains = n_q * hq;
  for (int i = tid; i < n_q * words; i += 1024) bm[i] = 0u;
  // page ids are loaded 8 at a time ahead of their LDS atomics; the first
  // batch is in flight during the query loads below
  // (n_q k_pages fits 32 bits: the bitmaps of a group fit in LDS)
  const uint32_t n_ids = static_cast<uint32_t>(n_q) * static_cast<uint32_t>(k_pages);
  const uint32_t kp32 = static_cast<uint32_t>(k_pages);
  int32_t pv[8];
  auto load_ids = [&](uint32_t i0) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * 1024 + tid;
      pv[u] = -1;
      if (i < n_ids) {
        const uint32_t t = i / kp32;
        pv[u] = pages[(static_cast<int64_t>(t) * hkv + g) * k_pages + (i - t * kp32)];
      }
    }
  };
  load_ids(0);
  // (d is 128, strides are multiples of 8 elements, base pointers 16-byte aligned)
  for (int i = tid; i < chains; i += 1024) {
    const int t = i / hq, h = i % hq;
    part[i] = sq_diff_sum<T>(qp + static_cast<int64_t>(i) * d, qc + t * am.q_st + h * am.q_sh, d);
  }
  __syncthreads();
  // the selection bitmaps of group g (as sel_prep_kernel)
  for (uint32_t i0 = 0; i0 < n_ids; i0 += 8 * 1024) {
    if (i0 > 0) load_ids(i0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * 1024 + tid;
      const uint32_t pg = static_cast<uint32_t>(pv[u]);
      if (i < n_ids && pg < static_cast<uint32_t>(n_pages))
        atomicOr(&bm[(i / kp32) * words + (pg >> 5)], 1u << (pg & 31));
    }
  }
  // the token classification
  for (int t = tid; t < n_q; t += 1024) {
    double total = 0.0;
    for (int h = 0; h < hq; ++h) total = total + part[t * hq + h];
    const double v = total / static_cast<double>(hq * d);
    mse_s[t] = v;
    if (g == 0 && am.mse) am.mse[t] = v;
  }
  __syncthreads();
  int rank = (am.pct * n_q + 99) / 100;
  if (rank < 1) rank = 1;
  for (int t = tid; t < n_q; t += 1024) {
    const double v = mse_s[t];
    int less = 0, leq = 0;
    for (int u = 0; u < n_q; ++u) {
      less += mse_s[u] < v ? 1 : 0;
      leq += mse_s[u] <= v ? 1 : 0;
    }
    if (less < rank && rank <= leq) cutoff_s = v;  // every writer writes the same value
  }
  __syncthreads();
  for (int t = tid; t < n_q; t += 1024) {
    const uint8_t a = mse_s[t] > cutoff_s ? 1 : 0;
    act_s[t] = a;
    if (g == 0) am.active[t] = a;
  }
  __syncthreads();
  for (int i = tid; i < n_q * words; i += 1024) {
    const int t = i / words, w = i % words;
    bitmap[(static_cast<int64_t>(t) * hkv + g) * words + w] = bm[i];
  }
  // the union over the active tokens, 256 words per pass
  const bool scanner = tid < 256;
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += 256) {
    const int w = w0 + tid;
    uint32_t u = 0u;
    if (scanner && w < words)
      for (int t = 0; t < n_q; ++t)
        if (act_s[t]) u |= bm[t * words + w];
    const int c = __popc(u);
    int total;
    const int incl = scan256(c, scan, total);
    int pos = base + (scanner ? incl : 0) - c;
    while (u) {
      const int b = __builtin_ctz(u);
      ulist[static_cast<int64_t>(g) * n_pages + pos++] = w * 32 + b;
      u &= u - 1;
    }
    base += total;
  }
  if (tid == 0) ucnt[g] = base;
}

// Both of the above in one launch when a KV group's bitmaps fit in LDS: one
// workgroup per g builds the rows (t, g) for every t, writes them, and (for
// GATHER) compacts their union over the active tokens.
constexpr int kPrepLdsWords = 12288;               // 48 KB of bitmap rows

__global__ __launch_bounds__(1024) void sel_prep_kernel(const int32_t* pages, int n_q, int hkv,
                                                       int k_pages, int words, int n_pages,
                                                       const uint8_t* active, int do_union,
                                                       uint32_t* bitmap, int32_t* ulist,
                                                       int32_t* ucnt) {
  extern __shared__ uint32_t bm[];                 // [n_q][words]
  __shared__ int scan[4];                          // wave totals of scan256
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  for (int i = tid; i < n_q * words; i += 1024) bm[i] = 0u;
  __syncthreads();
  // page ids are loaded 8 at a time ahead of their LDS atomics
  // (n_q k_pages fits 32 bits: the bitmaps of a group fit in LDS)
  const uint32_t n_ids = static_cast<uint32_t>(n_q) * static_cast<uint32_t>(k_pages);
  const uint32_t kp32 = static_cast<uint32_t>(k_pages);
  for (uint32_t i0 = 0; i0 < n_ids; i0 += 8 * 1024) {
    int32_t pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * 1024 + tid;
      pv[u] = -1;
      if (i < n_ids) {
        const uint32_t t = i / kp32;
        pv[u] = pages[(static_cast<int64_t>(t) * hkv + g) * k_pages + (i - t * kp32)];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = i0 + u * 1024 + tid;
      const uint32_t pg = static_cast<uint32_t>(pv[u]);
      if (i < n_ids && pg < static_cast<uint32_t>(n_pages))
        atomicOr(&bm[(i / kp32) * words + (pg >> 5)], 1u << (pg & 31));
    }
  }
  __syncthreads();
  for (int i = tid; i < n_q * words; i += 1024) {
    const int t = i / words, w = i % words;
    bitmap[(static_cast<int64_t>(t) * hkv + g) * words + w] = bm[i];
  }
  if (!do_union) return;                           // (uniform)
  // the union, 256 words per pass; threads past 256 only keep the barriers
  const bool scanner = tid < 256;
  int base = 0;
  for (int w0 = 0; w0 < words; w0 += 256) {
    const int w = w0 + tid;
    uint32_t u = 0u;
    if (scanner && w < words)
      for (int t = 0; t < n_q; ++t)
        if (!active || active[t]) u |= bm[t * words + w];
    const int c = __popc(u);
    int total;
    const int incl = scan256(c, scan, total);
    int pos = base + (scanner ? incl : 0) - c;
    while (u) {
      const int b = __builtin_ctz(u);
      ulist[static_cast<int64_t>(g) * n_pages + pos++] = w * 32 + b;
      u &= u - 1;
    }
    base += total;
  }
  if (tid == 0) ucnt[g] = base;
}

// Exclusive prefix sum of c over the NT threads of the workgroup (exact
// integers), by wave shuffles and one exchange of the wave totals in wsum
// (NT / 64 entries); total = the sum over all threads. Every thread calls it;
// it holds two barriers.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int c, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    pre += w < wave ? wsum[w] : 0;
    tot += wsum[w];
  }
  total = tot;
  __syncthreads();
  return x - c + pre;
}

constexpr int kUnionWords = 1024;            // union bitmaps a GATHER workgroup builds itself
constexpr int kClassifyTokens = 64;          // tokens it classifies itself

// ---------------------------------------------------------------------------
// The sparse MFMA pass.
// ---------------------------------------------------------------------------
struct SpTile {             // one tile in flight: K/V rows + where its halves are
  u32x4 k[8], v[8];
  int32_t page[2];          // page of each 16-key half
  int32_t valid[2];         // keys of each half that exist (0..16)
  uint32_t word[2];         // this lane's row bitmap word holding page[h]
};

__device__ __forceinline__ void softmax_set(const float (&x)[16], float c, float& m_run,
                                            float& l_run, f32x16 (&o)[4], bf16x8 (&ph)[2],
                                            bf16x8 (&pl)[2]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
  const bool bump = mx > m_run + kRescaleLog2;
  float alpha = 1.f;
  if (bump) {
    alpha = fast_exp2(m_run - mx);
    m_run = mx;
  }
  const float nm = m_run == kNegInf ? 0.f : -m_run;
  float psum = 0.f;
#pragma unroll
  for (int hj = 0; hj < 2; ++hj) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = fast_exp2(__builtin_fmaf(x[8 * hj + e], c, nm));
      psum += pf[e];
    }
    const bf16x8 hi = __builtin_convertvector(pf, bf16x8);
    ph[hj] = hi;
    pl[hj] = bf16_lo_part(pf, hi);
  }
  l_run = l_run * alpha + psum;
  if (__any(bump)) {
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
  }
}

// SPLIT keeps two O states (4 waves, one per SIMD: the register file holds
// both); GATHER runs FB_SPARSE_GATHER_WAVES waves, each with its own tile in
// flight (8 measured no faster than 4).
// (GATHER is built for two workgroups per CU: a 256-register budget keeps
// every value in VGPRs -- with a larger one the compiler parks state in
// AGPRs and reads it back every tile.)
template <bool SPLIT>
__global__ __launch_bounds__(64 * (SPLIT ? kSplitWaves : kGatherWaves),
                             (SPLIT || kGatherWaves > 4) ? 1 : 2)
void sparse_mfma_kernel(PrefixParams p) {
  constexpr int NSET = SPLIT ? 2 : 1;
  constexpr int kWaves = SPLIT ? kSplitWaves : kGatherWaves;
  constexpr int NT = 64 * kWaves;                  // threads
  constexpr int kStage = kWaves * kWaveLds;
  constexpr int kMerge = kWaves * 32 * kMergeStride * 4;
  constexpr int kLds = kMerge > kStage ? kMerge : kStage;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ float ml_s[kWaves][32][2];
  __shared__ int32_t upage[kMaxSlicePages];        // GATHER: this chunk's union pages

  int chunk, g, slab;
  {
    const int id = blockIdx.x;
    const int tq = id >> 3;
    slab = tq % p.n_slabs;
    const int idx = (tq / p.n_slabs) * 8 + (id & 7);
    if (idx >= p.n_chunks * p.hkv) return;
    chunk = idx % p.n_chunks;
    g = idx / p.n_chunks;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, r32 = lane & 31;
  const int G = p.group;
  const int R = p.n_q * G;
  const int row = slab * 32 + r32;
  const bool row_ok = row < R;
  const int t_row = row_ok ? row / G : 0;
  const int hpp = p.page_size >> 4;                // 16-key halves per page

  // GATHER with caller-built bitmaps: the token classification (optional)
  // and the union over the active tokens, in this workgroup, before the
  // tile LDS is first written (its space serves as scratch here)
  __shared__ uint8_t act_s[kClassifyTokens];
  __shared__ int wsum_s[kWaves];
  __shared__ int utot_s;
  uint32_t* ubits = reinterpret_cast<uint32_t*>(lds);               // [words]
  int* upre = reinterpret_cast<int*>(lds) + kUnionWords;            // [words]
  if (!SPLIT && p.union_from_bitmap) {
    if (p.classify) {
      // query MSE per token: per (token, head) four float64 sums of
      // (cur - prev)^2 over 32 dims each, in dim order, combined in quarter
      // order, the heads' sums in head order, / (Hq d) (no contraction);
      // nearest-rank cutoff; active iff above it. Every workgroup computes
      // the same bits; workgroup 0 writes them out.
      double* part = reinterpret_cast<double*>(lds + 2 * kUnionWords * 4);   // [n_q hq][4]
      double* mse_s = part + 4 * p.n_q * p.am.hq;                            // [n_q]
      const int hq = p.am.hq;
      const int items = 4 * p.n_q * hq;
      for (int i = tid; i < items; i += NT) {
        const int c = i >> 2, qd = i & 3;
        const int t = c / hq, h = c % hq;
        const int64_t po = static_cast<int64_t>(c) * kD + 32 * qd;
        const int64_t co = t * p.am.q_st + h * p.am.q_sh + 32 * qd;
        part[i] = p.am.dt == FB_BF16
                      ? sq_diff_sum32<uint16_t>(static_cast<const uint16_t*>(p.am.q_prev) + po,
                                                static_cast<const uint16_t*>(p.am.q_cur) + co)
                      : sq_diff_sum32<float>(static_cast<const float*>(p.am.q_prev) + po,
                                             static_cast<const float*>(p.am.q_cur) + co);
      }
      __syncthreads();
      {
#pragma clang fp contract(off)
        for (int t = tid; t < p.n_q; t += NT) {
          double total = 0.0;
          for (int h = 0; h < hq; ++h) {
            const double* q4 = part + 4 * (t * hq + h);
            const double ch = ((q4[0] + q4[1]) + q4[2]) + q4[3];
            total = total + ch;
          }
          mse_s[t] = total / static_cast<double>(hq * kD);
        }
      }
      __syncthreads();
      int rank = (p.am.pct * p.n_q + 99) / 100;
      if (rank < 1) rank = 1;
      double cut = 0.0;
      for (int t = 0; t < p.n_q; ++t) {              // every thread finds the same cutoff
        const double v = mse_s[t];
        int less = 0, leq = 0;
        for (int u = 0; u < p.n_q; ++u) {
          less += mse_s[u] < v ? 1 : 0;
          leq += mse_s[u] <= v ? 1 : 0;
        }
        if (less < rank && rank <= leq) cut = v;
      }
      for (int t = tid; t < p.n_q; t += NT) {
        const uint8_t a = mse_s[t] > cut ? 1 : 0;
        act_s[t] = a;
        if (blockIdx.x == 0) {
          p.am.active[t] = a;
          if (p.am.mse) p.am.mse[t] = mse_s[t];
        }
      }
    } else {
      for (int t = tid; t < p.n_q; t += NT) act_s[t] = (!p.active || p.active[t]) ? 1 : 0;
    }
    const int words = p.words;
    for (int wd = tid; wd < words; wd += NT) ubits[wd] = 0u;
    __syncthreads();
    // union words of group g over the active tokens: every (token, word)
    // load in flight at once, folded into LDS
    {
      const int n_ld = p.n_q * words;
      constexpr int kU = 8;
      for (int i0 = 0; i0 < n_ld; i0 += kU * NT) {
        uint32_t v[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = i0 + u * NT + tid;
          const int t = i < n_ld ? i / words : 0, wd = i - t * words;
          v[u] = (i < n_ld && act_s[t])
                     ? p.bitmap[(static_cast<int64_t>(t) * p.hkv + g) * words + wd] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int i = i0 + u * NT + tid;
          if (i < n_ld && v[u]) atomicOr(&ubits[i % words], v[u]);
        }
      }
    }
    __syncthreads();
    // popcounts' exclusive prefix over the words
    const int per = (words + NT - 1) / NT;           // consecutive words per thread
    int c = 0;
    for (int k = 0; k < per; ++k) {
      const int wd = tid * per + k;
      if (wd < words) c += __popc(ubits[wd]);
    }
    int total;
    int pre = block_excl_scan<NT>(c, wsum_s, total);
    for (int k = 0; k < per; ++k) {
      const int wd = tid * per + k;
      if (wd < words) {
        upre[wd] = pre;
        pre += __popc(ubits[wd]);
      }
    }
    if (tid == 0) utot_s = total;
    __syncthreads();
  }
  auto tok_on = [&](int t) -> bool {
    if (SPLIT) return true;
    if (p.union_from_bitmap) return act_s[t] != 0;
    return !p.active || p.active[t] != 0;
  };
  const bool row_on = row_ok && tok_on(t_row);

  // tiles of this group: all keys (SPLIT) or the union of selected pages
  int64_t n_vt;
  const int32_t* ulist = nullptr;
  int64_t n_half = 0;
  if (SPLIT) {
    n_vt = (p.n_kv + kTile - 1) / kTile;
  } else {
    n_half = static_cast<int64_t>(p.union_from_bitmap ? utot_s : p.ucnt[g]) * hpp;
    n_vt = (n_half + 1) / 2;
    if (!p.union_from_bitmap) ulist = p.ulist + static_cast<int64_t>(g) * p.n_pages;
  }
  // GATHER: the planned chunks share the actual union (no more tiles each
  // than planned for a union of every page)
  const int64_t tpc = SPLIT ? p.tiles_per_chunk : (n_vt + p.n_chunks - 1) / p.n_chunks;
  const int64_t vt_begin = static_cast<int64_t>(chunk) * tpc;
  const int64_t vt_end = vt_begin + tpc < n_vt ? vt_begin + tpc : n_vt;

  auto out_row = [&](int r, int set) -> int64_t {
    const RowOut& out = set == 0 ? p.out : p.out_res;
    const int t = r / G, h = g * G + r % G;
    return static_cast<int64_t>(chunk) * out.chunk_stride_rows + static_cast<int64_t>(t) * p.hq + h;
  };
  auto row_written = [&](int r) -> bool {
    if (r >= R) return false;
    return tok_on(r / G);
  };

  if (vt_begin >= vt_end) {                        // (GATHER) nothing to read: identity partial
    for (int e = tid; e < 32 * kD; e += NT) {
      const int r = slab * 32 + e / kD;
      if (row_written(r)) p.out.a[out_row(r, 0) * kD + e % kD] = 0.f;
    }
    for (int r0 = tid; r0 < 32; r0 += NT) {
      const int r = slab * 32 + r0;
      if (row_written(r)) p.out.l[out_row(r, 0)] = kNegInf;
    }
    return;
  }

  // GATHER: the chunk's slice of the union page list, staged in LDS
  const int64_t slice0 = SPLIT ? 0 : (2 * vt_begin) / hpp;
  if (!SPLIT) {
    int64_t slice1 = (2 * vt_end - 1) / hpp;         // inclusive, within the union
    slice1 = slice1 < (n_half - 1) / hpp ? slice1 : (n_half - 1) / hpp;
    if (p.union_from_bitmap) {
      // the union pages of rank slice0 .. slice1, from the words that hold them
      const int s0 = static_cast<int>(slice0), s1 = static_cast<int>(slice1);
      for (int wd = tid; wd < p.words; wd += NT) {
        int r = upre[wd];
        uint32_t u = ubits[wd];
        if (r > s1 || r + __popc(u) <= s0) continue;
        while (u) {
          const int b = __builtin_ctz(u);
          if (r >= s0 && r <= s1) upage[r - s0] = wd * 32 + b;
          ++r;
          u &= u - 1;
        }
      }
    } else {
      for (int64_t i = tid; i <= slice1 - slice0; i += NT) upage[i] = ulist[slice0 + i];
    }
    __syncthreads();
  }

  // Q^T operand of this lane's row (zero for rows past R)
  bf16x8 qop[8];
  {
    const int jh = row_ok ? row % G : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + static_cast<int64_t>(t_row) * p.q_st +
                         static_cast<int64_t>(g * G + jh) * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qop[kk] = row_ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * hl) : bf16x8{};
  }
  const uint32_t* bm_row = p.bitmap + (static_cast<int64_t>(t_row) * p.hkv + g) * p.words;

  const char* kg = static_cast<const char*>(p.k) + static_cast<int64_t>(g) * p.kv_sh * 2;
  const char* vg = static_cast<const char*>(p.v) + static_cast<int64_t>(g) * p.kv_sh * 2;
  const int64_t kvst_b = p.kv_st * 2;
  const int lrow = lane >> 4, lpiece = lane & 15;
  char* kl = lds + w * kWaveLds;
  char* vl = kl + kKBytes;
  char* k_wr = kl + lrow * kKRow + lpiece * 16;
  char* v_wr = vl + lrow * kVRow + lpiece * 16;
  const char* k_rd = kl + r32 * kKRow + hl * 16;
  const int grp = lane >> 4, s4 = (lane & 15) >> 2, q4 = lane & 3;
  const char* v_rd = vl + (4 * (grp >> 1) + s4) * kVRow + 32 * (grp & 1) + 8 * q4;

  const int64_t vt_last = vt_end - 1;
  // token and page arithmetic in 32 bits (prefixes on this path hold fewer
  // than 2^31 keys), with no division for the usual 16-token pages
  const uint32_t n_pages32 = static_cast<uint32_t>(p.n_pages);
  const uint32_t ps32 = static_cast<uint32_t>(p.page_size);
  const uint32_t hpp32 = static_cast<uint32_t>(hpp);
  const uint32_t slice0_32 = static_cast<uint32_t>(slice0);
  auto load_tile = [&](int64_t vt64) -> SpTile {
    SpTile r;
    const uint32_t vt = static_cast<uint32_t>(vt64 < vt_last ? vt64 : vt_last);
    int64_t tok0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t tok;
      int32_t page;
      bool exists;
      if (SPLIT) {
        const uint32_t t32 = vt * kTile + 16 * h;
        const uint32_t pg = hpp32 == 1 ? t32 >> 4 : t32 / ps32;   // (past n_kv: no keys, any bit)
        page = static_cast<int32_t>(pg < n_pages32 ? pg : n_pages32 - 1);
        tok = t32;
        exists = true;
      } else {
        uint32_t hx = 2 * vt + h;
        exists = hx < static_cast<uint64_t>(n_half);
        hx = exists ? hx : 2 * vt;
        if (hpp32 == 1) {
          page = upage[hx - slice0_32];
          tok = static_cast<int64_t>(static_cast<uint32_t>(page) * ps32);
        } else {
          const uint32_t q = hx / hpp32;
          page = upage[q - slice0_32];
          tok = static_cast<int64_t>(static_cast<uint32_t>(page) * ps32 + 16 * (hx - q * hpp32));
        }
      }
      const int64_t rem = p.n_kv - tok;
      r.valid[h] = !exists || rem <= 0 ? 0 : (rem < 16 ? static_cast<int32_t>(rem) : 16);
      r.page[h] = page;
      tok0[h] = tok;
      r.word[h] = row_on ? bm_row[page >> 5] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t tok = tok0[i >> 2] + 4 * (i & 3) + lrow;
      tok = tok < p.n_kv ? tok : p.n_kv - 1;
      const int64_t off = tok * kvst_b + lpiece * 16;
      // streamed once: non-temporal, so the reads do not allocate in the
      // last-level cache (and evict the dirty lines other work left there)
      r.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kg + off));
      r.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vg + off));
    }
    return r;
  };

  f32x16 o[NSET][4];
  float m_run[NSET], l_run[NSET];
#pragma unroll
  for (int s = 0; s < NSET; ++s) {
    m_run[s] = kNegInf;
    l_run[s] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[s][db] = f32x16{};
  }

  auto process = [&](const SpTile& tl) {
    f32x16 sc = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      sc = mfma32(*reinterpret_cast<const bf16x8*>(k_rd + 32 * kk), qop[kk], sc);
    const bool sel0 = (tl.word[0] >> (tl.page[0] & 31)) & 1u;
    const bool sel1 = (tl.word[1] >> (tl.page[1] & 31)) & 1u;
    float xs[16], xr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int h = i >> 3;                        // half of the tile
      const int kh = 8 * ((i >> 2) & 1) + 4 * hl + (i & 3);   // key within the half
      const bool val = row_on && kh < tl.valid[h];
      const bool sel = h ? sel1 : sel0;
      xs[i] = val && sel ? sc[i] : kNegInf;
      if (SPLIT) xr[i] = val && !sel ? sc[i] : kNegInf;
    }
    bf16x8 ph[NSET][2], pl[NSET][2];
    softmax_set(xs, p.scale_log2, m_run[0], l_run[0], o[0], ph[0], pl[0]);
    if (SPLIT) softmax_set(xr, p.scale_log2, m_run[NSET - 1], l_run[NSET - 1], o[NSET - 1],
                                 ph[NSET - 1], pl[NSET - 1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x4 v0 = ds_read_tr(v_rd + (16 * j) * kVRow + 64 * db);
        const bf16x4 v1 = ds_read_tr(v_rd + (16 * j + 8) * kVRow + 64 * db);
        va[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int s = 0; s < NSET; ++s) {
#pragma unroll
        for (int db = 0; db < 4; ++db) o[s][db] = mfma32(va[db], ph[s][j], o[s][db]);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[s][db] = mfma32(va[db], pl[s][j], o[s][db]);
      }
    }
    asm volatile("" ::: "memory");
  };

  auto stage = [&](const SpTile& tl) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(k_wr + 4 * i * kKRow) = tl.k[i];
      *reinterpret_cast<u32x4*>(v_wr + 4 * i * kVRow) = tl.v[i];
    }
    asm volatile("" ::: "memory");
  };
  if (SPLIT || FB_SPARSE_PREFETCH < 2) {
    SpTile cur = load_tile(vt_begin + w);
    for (int64_t vt = vt_begin + w; vt < vt_end; vt += kWaves) {
      stage(cur);
      const SpTile nxt = load_tile(vt + kWaves);
      process(cur);
      cur = nxt;
    }
  } else {
    // two tiles in flight while one is processed: three register sets in
    // rotation, the loop unrolled by three (loads past the chunk's last tile
    // re-read it: load_tile clamps)
    constexpr int K = kWaves;
    SpTile ta = load_tile(vt_begin + w), tb = load_tile(vt_begin + w + K), tc;
    for (int64_t vt = vt_begin + w; vt < vt_end; vt += 3 * K) {
      stage(ta);
      tc = load_tile(vt + 2 * K);
      process(ta);
      if (vt + K >= vt_end) break;
      stage(tb);
      ta = load_tile(vt + 3 * K);
      process(tb);
      if (vt + 2 * K >= vt_end) break;
      stage(tc);
      tb = load_tile(vt + 4 * K);
      process(tc);
    }
  }

  // ---- merge the four waves' states through LDS, write the chunk partial --
#pragma unroll
  for (int s = 0; s < NSET; ++s) {
    const float lsum = l_run[s] + __shfl_xor(l_run[s], 32, 64);
    __syncthreads();                               // tile LDS (or the previous set) no longer read
    if (hl == 0) {
      ml_s[w][r32][0] = m_run[s];
      ml_s[w][r32][1] = lsum;
    }
    __syncthreads();
    float* mg = reinterpret_cast<float*>(lds);
    {
      float M = kNegInf;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, ml_s[ww][r32][0]);
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = ml_s[ww][r32][0];
        if (mw != kNegInf) tot += ml_s[ww][r32][1] * fast_exp2(mw - M);
      }
      const float f = (m_run[s] == kNegInf || tot == 0.f) ? 0.f : fast_exp2(m_run[s] - M) / tot;
      float* dst = mg + (w * 32 + r32) * kMergeStride;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[32 * db + 8 * (i >> 2) + 4 * hl + (i & 3)] = o[s][db][i] * f;
    }
    __syncthreads();
    const RowOut& out = s == 0 ? p.out : p.out_res;
    for (int e = tid; e < 32 * kD; e += NT) {
      const int r = e / kD, c = e % kD;
      if (!row_written(slab * 32 + r)) continue;
      float sum = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) sum += mg[(ww * 32 + r) * kMergeStride + c];
      out.a[out_row(slab * 32 + r, s) * kD + c] = sum;
    }
    for (int r = tid; r < 32; r += NT) {
      if (!row_written(slab * 32 + r)) continue;
      float M = kNegInf;
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, ml_s[ww][r][0]);
      float tot = 0.f;
      for (int ww = 0; ww < kWaves; ++ww) {
        const float mw = ml_s[ww][r][0];
        if (mw != kNegInf) tot += ml_s[ww][r][1] * fast_exp2(mw - M);
      }
      out.l[out_row(slab * 32 + r, s)] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
    }
  }
}

}  // namespace

hipError_t launch_sel_bitmap(const int32_t* pages, int n_rows, int k_pages, int words, int n_pages,
                             uint32_t* bitmap, hipStream_t s) {
  hipLaunchKernelGGL(sel_bitmap_kernel, dim3(n_rows), dim3(256), words * sizeof(uint32_t), s, pages,
                     k_pages, words, n_pages, bitmap);
  return hipGetLastError();
}

// the workgroup keeps the union words and every token's active flag in LDS
bool gather_union_fits(int n_q, int words) {
  return words >= 1 && words <= kUnionWords && n_q >= 1 && n_q <= kClassifyTokens;
}

bool gather_classify_fits(int n_q, int hq) {
  // the float64 sums of the classification (four per token and head, then
  // one per token) in the tile LDS after the union words
  const size_t need = 2 * kUnionWords * 4 + (4 * static_cast<size_t>(n_q) * hq + n_q) * sizeof(double);
  return n_q >= 1 && n_q <= kClassifyTokens && need <= static_cast<size_t>(kGatherWaves) * kWaveLds;
}

bool sel_prep_fits(int n_q, int words) {
  return static_cast<int64_t>(n_q) * words <= kPrepLdsWords;
}

hipError_t launch_sel_prep(const int32_t* pages, int n_q, int hkv, int k_pages, int words,
                           int n_pages, const uint8_t* active, int do_union, uint32_t* bitmap,
                           int32_t* ulist, int32_t* ucnt, hipStream_t s) {
  hipLaunchKernelGGL(sel_prep_kernel, dim3(hkv), dim3(1024), static_cast<size_t>(n_q) * words * 4, s,
                     pages, n_q, hkv, k_pages, words, n_pages, active, do_union, bitmap, ulist,
                     ucnt);
  return hipGetLastError();
}

static size_t sel_prep_mse_lds(int n_q, int hq, int words) {
  return (static_cast<size_t>((n_q * words + 1) & ~1) * 4) +
         (static_cast<size_t>(n_q) * hq + n_q) * sizeof(double);
}

bool sel_prep_mse_fits(int n_q, int hq, int words) {
  return n_q >= 1 && n_q <= 1024 && sel_prep_mse_lds(n_q, hq, words) <= 64 * 1024;
}

hipError_t launch_sel_prep_mse(const int32_t* pages, int n_q, int hkv, int k_pages, int words,
                               int n_pages, const ActiveFromMse& am, uint32_t* bitmap,
                               int32_t* ulist, int32_t* ucnt, hipStream_t s) {
  if (am.d != 128) return hipErrorInvalidValue;
  const size_t lds = sel_prep_mse_lds(n_q, am.hq, words);
  if (am.dt == FB_BF16)
    hipLaunchKernelGGL(sel_prep_mse_kernel<uint16_t>, dim3(hkv), dim3(1024), lds, s, pages, n_q,
                       hkv, k_pages, words, n_pages, am, bitmap, ulist, ucnt);
  else
    hipLaunchKernelGGL(sel_prep_mse_kernel<float>, dim3(hkv), dim3(1024), lds, s, pages, n_q, hkv,
                       k_pages, words, n_pages, am, bitmap, ulist, ucnt);
  return hipGetLastError();
}

hipError_t launch_sel_union(const uint32_t* bitmap, const uint8_t* active, int n_q, int hkv,
                            int words, int32_t* ulist, int32_t* ucnt, int n_pages, hipStream_t s) {
  hipLaunchKernelGGL(sel_union_kernel, dim3(hkv), dim3(256), 0, s, bitmap, active, n_q, hkv, words,
                     ulist, ucnt, n_pages);
  return hipGetLastError();
}

// a chunk of n tiles spans at most 2n union pages (one per 16-key half)
int sparse_max_tiles_per_chunk() { return (kMaxSlicePages - 2) / 2; }

hipError_t launch_prefix_sparse(const PrefixParams& p, hipStream_t s) {
  const int n_cg = p.n_chunks * p.hkv;
  const dim3 grid(static_cast<unsigned>((n_cg + 7) / 8 * 8 * p.n_slabs));
  if (p.sel_mode == FB_SEL_SPLIT)
    hipLaunchKernelGGL(sparse_mfma_kernel<true>, grid, dim3(64 * kSplitWaves), 0, s, p);
  else
    hipLaunchKernelGGL(sparse_mfma_kernel<false>, grid, dim3(64 * kGatherWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace fb
