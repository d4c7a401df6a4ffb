// k4_pages.hip -- QUEST-style page selection for the sparse subsystem.
//
// LoSA (Locality Aware Sparse Attention for Block-Wise Diffusion Language
// Models), s2: active block tokens attend only to the prefix pages a QUEST
// selector picks; FlashBlock technical summary, s2 sparse compatibility: the
// pages left out form the residual whose contribution is cached.
//
// The pages name QUEST without restating it; the selector here is the page
// bound: per (KV head, page, dim) the min and max of the page's keys, and for
// a query row the upper bound sum_d max(q_d kmin_d, q_d kmax_d) of q.k over
// the page, maximised over the query heads of the KV group. Products of two
// bf16 (or two fp32) values are exact in float64, and the sum runs
// sequentially over d with contraction disabled, so the bound's bits do not
// depend on the device. Top-k is exact: the k-th largest key is found by
// bisection on an order-preserving 64-bit image of the bound, ties go to the
// lower page id, and the chosen pages are emitted in ascending order.
#include "fb_internal.h"

#include <math.h>

namespace fb {
namespace {

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// Element e of a 16-byte group of bf16 (8) or fp32 (4) values, as float.
template <typename T> __device__ __forceinline__ float grp_float(u32x4v w, int e);
template <> __device__ __forceinline__ float grp_float<uint16_t>(u32x4v w, int e) {
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
}
template <> __device__ __forceinline__ float grp_float<float>(u32x4v w, int e) {
  return __uint_as_float(w[e]);
}

// kmin/kmax[g][p][c] over the tokens of page p (the last page may be short),
// for pages p0 .. p0 + n_pg - 1; page_cap pages per KV head in storage. One
// thread per (page, 16-byte group of dims): it walks the page's tokens with
// 16-byte loads and writes its groups of kmin and kmax with 16-byte stores
// (the min and max of bf16 or fp32 values are themselves exact values).
template <typename T>
__global__ __launch_bounds__(256) void page_meta_kernel(const T* k, int64_t kv_st, int64_t kv_sh,
                                                        int64_t n_kv, int d, int page_size,
                                                        int64_t p0, int64_t n_pg, int64_t page_cap,
                                                        T* kmin, T* kmax) {
  constexpr int NE = 16 / sizeof(T);
  const int gpr = d / NE;                          // groups per row
  const int g = blockIdx.y;
  const int64_t v = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (v >= n_pg * gpr) return;
  const int64_t p = p0 + v / gpr;
  const int cg = static_cast<int>(v % gpr) * NE;
  const int64_t lo = p * page_size;
  const int64_t hi = lo + page_size < n_kv ? lo + page_size : n_kv;
  float mn[NE], mx[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    mn[e] = __builtin_huge_valf();
    mx[e] = -__builtin_huge_valf();
  }
  const T* base = k + static_cast<int64_t>(g) * kv_sh + cg;
  for (int64_t t = lo; t < hi; ++t) {
    const u32x4v w = *reinterpret_cast<const u32x4v*>(base + t * kv_st);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float x = grp_float<T>(w, e);
      mn[e] = fminf(mn[e], x);
      mx[e] = fmaxf(mx[e], x);
    }
  }
  u32x4v a, b;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (NE == 8) {                                 // bf16: the high halves of the floats
      a[c] = (__float_as_uint(mn[2 * c]) >> 16) | (__float_as_uint(mn[2 * c + 1]) & 0xffff0000u);
      b[c] = (__float_as_uint(mx[2 * c]) >> 16) | (__float_as_uint(mx[2 * c + 1]) & 0xffff0000u);
    } else {
      a[c] = __float_as_uint(mn[c]);
      b[c] = __float_as_uint(mx[c]);
    }
  }
  const int64_t o = (static_cast<int64_t>(g) * page_cap + p) * d + cg;
  *reinterpret_cast<u32x4v*>(kmin + o) = a;
  *reinterpret_cast<u32x4v*>(kmax + o) = b;
}

// bound[t][g][p]: one thread per (page, token). The query rows of the
// workgroup's tokens (tc of them, from blockIdx.z * tc) and the page block's
// metadata sit in LDS as float (exact copies of the inputs).
constexpr int kPagesPerBlock = 32;

template <typename T>
__global__ __launch_bounds__(256) void page_bound_kernel(const T* q, int64_t q_st, int64_t q_sh,
                                                         const T* kmin, const T* kmax, int n_q,
                                                         int tc, int hq, int hkv, int d,
                                                         int64_t n_pages, int64_t page_cap,
                                                         const uint8_t* active, double* bound) {
#pragma clang fp contract(off)
  extern __shared__ float sm[];
  const int G = hq / hkv;
  const int g = blockIdx.y;
  const int t0 = blockIdx.z * tc;
  const int nt = n_q - t0 < tc ? n_q - t0 : tc;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPagesPerBlock;
  const int np = n_pages - p0 < kPagesPerBlock ? static_cast<int>(n_pages - p0) : kPagesPerBlock;
  // page rows padded to d + 1 floats: the 32 pages a wave reads at once fall
  // in distinct LDS banks
  const int ds = d + 1;
  float* qs = sm;                                    // [tc][G][d]
  float* mn = qs + tc * G * d;                       // [kPagesPerBlock][d + 1]
  float* mx = mn + kPagesPerBlock * ds;
  for (int e = threadIdx.x; e < nt * G * d; e += blockDim.x) {
    const int t = e / (G * d), j = (e / d) % G, c = e % d;
    qs[e] = ldf<T>(q + static_cast<int64_t>(t0 + t) * q_st + static_cast<int64_t>(g * G + j) * q_sh + c);
  }
  for (int e = threadIdx.x; e < np * d; e += blockDim.x) {
    const int64_t o = (static_cast<int64_t>(g) * page_cap + p0) * d + e;
    const int ls = (e / d) * ds + e % d;
    mn[ls] = ldf<T>(kmin + o);
    mx[ls] = ldf<T>(kmax + o);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < np * nt; e += blockDim.x) {
    const int pi = e % np, tl = e / np, t = t0 + tl;
    if (active && !active[t]) continue;
    double best = -__builtin_huge_val();
    for (int j = 0; j < G; ++j) {
      const float* qr = qs + (tl * G + j) * d;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) {
        const double qv = qr[c];
        const double lo = qv * static_cast<double>(mn[pi * ds + c]);
        const double hi = qv * static_cast<double>(mx[pi * ds + c]);
        acc = acc + (lo > hi ? lo : hi);
      }
      best = acc > best ? acc : best;
    }
    bound[(static_cast<int64_t>(t) * hkv + g) * n_pages + p0 + pi] = best;
  }
}

// Same bound, with the G query heads of the group as G independent chains
// (the sum of each head still runs sequentially over d, so every bit equals
// the one-head-at-a-time kernel's). Each term is one select and one fused
// multiply-add: max(q a, q b) with a <= b is q b for q >= 0 and q a
// otherwise, and the product of two bf16 (or fp32) values is exact in
// float64, so acc + that product rounds once either way.
// Workgroup = (32 pages, KV group g, TC tokens). One round trip stages the
// page rows (kept in their own dtype in LDS: bf16 rows are half the size,
// so four workgroups fit on a CU), the TC tokens' query rows and their
// active flags; with an active mask only the active tokens are scored,
// packed onto the first threads.
template <typename T>
constexpr int bound_row_stride(int d) {            // LDS row of a page (elements)
  return sizeof(T) == 2 ? d + 4 : d + 1;           // bf16: 2-word bank step; fp32: 1
}

template <typename T, int G, int TC>
__global__ __launch_bounds__(256) void page_bound_g_kernel(const T* q, int64_t q_st, int64_t q_sh,
                                                           const T* kmin, const T* kmax, int n_q,
                                                           int hkv, int d, int64_t n_pages,
                                                           int64_t page_cap, const uint8_t* active,
                                                           double* bound) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  __shared__ int tok[TC];
  __shared__ int n_tok_s;
  const int g = blockIdx.y;
  const int t0 = blockIdx.z * TC;
  const int nt_all = n_q - t0 < TC ? n_q - t0 : TC;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPagesPerBlock;
  const int np = n_pages - p0 < kPagesPerBlock ? static_cast<int>(n_pages - p0) : kPagesPerBlock;
  const int rs = bound_row_stride<T>(d);
  float* qs = sm;                                    // [TC][d][G] (heads innermost)
  T* mn = reinterpret_cast<T*>(qs + TC * G * d);     // [kPagesPerBlock][rs]
  T* mx = mn + kPagesPerBlock * rs;
  // wave 0 compacts the active tokens (one flag load per lane, a ballot and
  // a prefix count) while every thread stages rows
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const bool on = lane < nt_all && (!active || active[t0 + lane]);
    const unsigned long long m = __ballot(on);
    if (on) tok[__popcll(m & ((1ull << lane) - 1ull))] = lane;
    if (lane == 0) n_tok_s = __popcll(m);
  }
  // 16-byte loads (rows of d elements, 16-byte aligned: the host checks the
  // bases, strides are multiples of 8 elements)
  constexpr int NE = 16 / sizeof(T);
  const int gpr = d / NE;                            // 16-byte groups per row
  for (int v = threadIdx.x; v < np * gpr; v += blockDim.x) {
    const int pi = v / gpr, cg = (v % gpr) * NE;
    const int64_t o = (static_cast<int64_t>(g) * page_cap + p0 + pi) * d + cg;
    const u32x4v a = *reinterpret_cast<const u32x4v*>(kmin + o);
    const u32x4v b = *reinterpret_cast<const u32x4v*>(kmax + o);
    uint32_t* wa = reinterpret_cast<uint32_t*>(mn + pi * rs + cg);
    uint32_t* wb = reinterpret_cast<uint32_t*>(mx + pi * rs + cg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wa[e] = a[e];
      wb[e] = b[e];
    }
  }
  for (int v = threadIdx.x; v < nt_all * G * gpr; v += blockDim.x) {
    const int row = v / gpr, cg = (v % gpr) * NE;
    const int t = row / G, j = row % G;
    const u32x4v w = *reinterpret_cast<const u32x4v*>(
        q + static_cast<int64_t>(t0 + t) * q_st + static_cast<int64_t>(g * G + j) * q_sh + cg);
#pragma unroll
    for (int e = 0; e < NE; ++e) qs[(t * d + cg + e) * G + j] = grp_float<T>(w, e);
  }
  __syncthreads();
  const int nt = n_tok_s;
  for (int e = threadIdx.x; e < np * nt; e += blockDim.x) {
    const int pi = e % np, tl = tok[e / np];
    const float* qr = qs + tl * G * d;
    double acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.0;
    if constexpr (sizeof(T) == 2) {                  // two dims per LDS word
      // 8 dims per step: the page's kmin / kmax words (two 8-byte reads
      // each) and the token's 8 x G query values (2 G 16-byte reads) are
      // read before the step's multiply-adds, and the next step's reads are
      // issued before them (the LDS latency is otherwise paid per read)
      const uint32_t* mnw = reinterpret_cast<const uint32_t*>(mn + pi * rs);
      const uint32_t* mxw = reinterpret_cast<const uint32_t*>(mx + pi * rs);
      struct Chunk {
        uint2 a0, a1, b0, b1;
        float4 qv[2 * G];                            // [8 dims][G]
      };
      auto load = [&](int c8, Chunk& k) __attribute__((always_inline)) {
        k.a0 = *reinterpret_cast<const uint2*>(mnw + c8 / 2);
        k.a1 = *reinterpret_cast<const uint2*>(mnw + c8 / 2 + 2);
        k.b0 = *reinterpret_cast<const uint2*>(mxw + c8 / 2);
        k.b1 = *reinterpret_cast<const uint2*>(mxw + c8 / 2 + 2);
#pragma unroll
        for (int i = 0; i < 2 * G; ++i) k.qv[i] = *reinterpret_cast<const float4*>(qr + c8 * G + 4 * i);
      };
      auto step = [&](const Chunk& k) __attribute__((always_inline)) {
        const uint32_t wa[4] = {k.a0.x, k.a0.y, k.a1.x, k.a1.y};
        const uint32_t wb[4] = {k.b0.x, k.b0.y, k.b1.x, k.b1.y};
        const float* qf = reinterpret_cast<const float*>(k.qv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t ua = wa[e >> 1], ub = wb[e >> 1];
          const float av = __uint_as_float((e & 1) ? (ua & 0xffff0000u) : (ua << 16));
          const float bv = __uint_as_float((e & 1) ? (ub & 0xffff0000u) : (ub << 16));
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float qv = qf[e * G + j];
            acc[j] = __builtin_fma(static_cast<double>(qv),
                                   static_cast<double>(qv >= 0.f ? bv : av), acc[j]);
          }
        }
      };
      Chunk k0, k1;
      load(0, k0);
      for (int c8 = 0; c8 < d; c8 += 16) {           // (d is a multiple of 16)
        load(c8 + 8, k1);
        step(k0);
        if (c8 + 16 < d) load(c8 + 16, k0);
        step(k1);
      }
    } else {
      const float* mnr = reinterpret_cast<const float*>(mn) + pi * rs;
      const float* mxr = reinterpret_cast<const float*>(mx) + pi * rs;
      for (int c = 0; c < d; ++c) {
        const float a = mnr[c], b = mxr[c];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          const float qv = qr[c * G + j];
          acc[j] = __builtin_fma(static_cast<double>(qv), static_cast<double>(qv >= 0.f ? b : a),
                                 acc[j]);
        }
      }
    }
    double best = acc[0];
#pragma unroll
    for (int j = 1; j < G; ++j) best = acc[j] > best ? acc[j] : best;
    bound[(static_cast<int64_t>(t0 + tl) * hkv + g) * n_pages + p0 + pi] = best;
  }
}

// Order-preserving image of a double as an unsigned 64-bit key.
__device__ __forceinline__ uint64_t okey(double x) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(x));
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ int block_sum(int v, int* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = blockDim.x / 2; s >= 1; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  const int r = red[0];
  __syncthreads();
  return r;
}

// One workgroup per (token, KV head): exact top-k of bound[t][g][:].
__global__ __launch_bounds__(256) void page_topk_kernel(const double* bound, int hkv,
                                                        int64_t n_pages, int k,
                                                        const uint8_t* active, int32_t* pages,
                                                        uint8_t* flags) {
  __shared__ int red[256];
  __shared__ int scan[256];
  if (active && !active[blockIdx.x]) return;       // a row of an inactive token
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * hkv + blockIdx.y;
  const double* b = bound + row * n_pages;
  int32_t* out = pages + row * k;
  if (k <= 0) return;
  // T = the k-th largest key: the largest T with #{key >= T} >= k.
  uint64_t T = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    int c = 0;
    for (int64_t p = tid; p < n_pages; p += 256) c += okey(b[p]) >= cand ? 1 : 0;
    if (block_sum(c, red) >= k) T = cand;
  }
  int gt = 0;
  for (int64_t p = tid; p < n_pages; p += 256) gt += okey(b[p]) > T ? 1 : 0;
  const int n_gt = block_sum(gt, red);
  const int need_eq = k - n_gt;                      // >= 1 ties at T, lowest ids first
  // emit in ascending page order: tiles of 256 pages, block-wide prefix sums
  int written = 0, eq_taken = 0;
  for (int64_t base = 0; base < n_pages; base += 256) {
    const int64_t p = base + tid;
    int is_gt = 0, is_eq = 0;
    if (p < n_pages) {
      const uint64_t kk = okey(b[p]);
      is_gt = kk > T;
      is_eq = kk == T;
    }
    // inclusive scan of is_eq to rank the ties in this tile
    scan[tid] = is_eq;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {
      const int v = tid >= s ? scan[tid - s] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int eq_rank = eq_taken + scan[tid] - is_eq;    // ties before me
    const int tile_eq = scan[255];
    __syncthreads();
    const int sel = is_gt || (is_eq && eq_rank < need_eq);
    scan[tid] = sel;
    __syncthreads();
    for (int s = 1; s < 256; s <<= 1) {
      const int v = tid >= s ? scan[tid - s] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (sel) out[written + scan[tid] - 1] = static_cast<int32_t>(p);
    if (flags && p < n_pages) flags[row * n_pages + p] = sel ? 1 : 0;
    written += scan[255];
    eq_taken += tile_eq;
    __syncthreads();
  }
}

// Block-wide exclusive scan over 256 threads (4 waves).
__device__ __forceinline__ int block_exscan4(int v, int* red, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;                                       // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += red[i];
  total = red[0] + red[1] + red[2] + red[3];
  return before + x - v;
}

// Top-k with every key in registers: thread tid owns the KPT consecutive
// pages [tid * KPT, tid * KPT + KPT), so ascending emission needs one scan.
// Same result as page_topk_kernel: T = the k-th largest key, found exactly
// by an 8-pass radix select (8 bits per pass, most significant first: the
// pass's histogram over the keys that share T's prefix fixes the next byte),
// then every key > T and the lowest-id ties at T.
__device__ __forceinline__ int block_inscan4(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  for (int i = 0; i < w; ++i) x += red[i];
  return x;
}

template <int KPT>
__global__ __launch_bounds__(256) void page_topk_reg_kernel(const double* bound, int hkv,
                                                            int64_t n_pages, int k,
                                                            const uint8_t* active, int32_t* pages,
                                                            uint8_t* flags, uint32_t* bitmap) {
  __shared__ int hist[256];
  __shared__ int red[4];
  __shared__ unsigned long long sh_prefix;
  __shared__ int sh_kk, sh_h;
  if (active && !active[blockIdx.x]) return;       // a row of an inactive token
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * hkv + blockIdx.y;
  const double* b = bound + row * n_pages;
  int32_t* out = pages + row * k;
  const int64_t p0 = static_cast<int64_t>(tid) * KPT;
  uint64_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = p0 + i < n_pages ? okey(b[p0 + i]) : 0ull;
  // (okey of any bound is > 0; padding 0 is never in T's group, see below)

  // Leading bytes every key shares (from the keys' min and max) need no
  // histogram: they are T's bytes, and the group stays all keys.
  __shared__ unsigned long long sh_lo[4], sh_hi[4];
  uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (p0 + i < n_pages) {
      lo = key[i] < lo ? key[i] : lo;
      hi = key[i] > hi ? key[i] : hi;
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint64_t l2 = __shfl_xor(lo, o, 64), h2 = __shfl_xor(hi, o, 64);
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  if ((tid & 63) == 0) {
    sh_lo[tid >> 6] = lo;
    sh_hi[tid >> 6] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    lo = sh_lo[w] < lo ? sh_lo[w] : lo;
    hi = sh_hi[w] > hi ? sh_hi[w] : hi;
  }
  const uint64_t diff = lo ^ hi;
  const int first = diff ? __clzll(diff) / 8 : 8;  // leading bytes in common
  uint64_t pmask = first == 0 ? 0ull : (first == 8 ? ~0ull : ~0ull << (64 - 8 * first));
  uint64_t prefix = lo & pmask;
  int kk = k;                                      // rank of T within the current group
  int early = 0;                                   // 1: T = the group's max, 2: its min
  for (int pass = first; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (p0 + i < n_pages && (key[i] & pmask) == prefix)
        atomicAdd(&hist[(key[i] >> shift) & 255], 1);
    __syncthreads();
    // thread tid takes byte value bv = 255 - tid: S = #group keys with byte >= bv
    const int bv = 255 - tid;
    const int h = hist[bv];
    const int S = block_inscan4(h, red);
    if (S >= kk && S - h < kk) {                   // exactly one byte value
      sh_prefix = prefix | (static_cast<uint64_t>(bv) << shift);
      sh_kk = kk - (S - h);
      sh_h = h;
    }
    __syncthreads();
    prefix = sh_prefix;
    kk = sh_kk;
    pmask |= 255ull << shift;
    // T is the group's largest key when it takes rank 1 in it, its smallest
    // when it takes the last rank: one reduction ends the search
    if (kk == 1 || kk == sh_h) {
      early = kk == 1 ? 1 : 2;
      break;
    }
  }
  uint64_t T = prefix;
  if (early) {
    uint64_t v = early == 1 ? 0ull : ~0ull;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (p0 + i < n_pages && (key[i] & pmask) == prefix)
        v = early == 1 ? (key[i] > v ? key[i] : v) : (key[i] < v ? key[i] : v);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const uint64_t u = __shfl_xor(v, o, 64);
      v = early == 1 ? (u > v ? u : v) : (u < v ? u : v);
    }
    if ((tid & 63) == 0) sh_lo[tid >> 6] = v;
    __syncthreads();
    T = sh_lo[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) T = early == 1 ? (sh_lo[w] > T ? sh_lo[w] : T) : (sh_lo[w] < T ? sh_lo[w] : T);
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    gt += key[i] > T ? 1 : 0;
    eq += key[i] == T ? 1 : 0;
  }
  int tot;
  (void)block_exscan4(gt, red, tot);
  const int need_eq = k - tot;                     // ties at T to take, lowest ids first
  const int eq_before = block_exscan4(eq, red, tot);
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  int pos = block_exscan4(gt + take_eq, red, tot);
  int eq_seen = 0;
  uint32_t bits = 0;                               // bit i: page p0 + i chosen
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool is_eq = key[i] == T;
    const bool sel = key[i] > T || (is_eq && eq_seen < take_eq);
    eq_seen += is_eq ? 1 : 0;
    if (sel) out[pos++] = static_cast<int32_t>(p0 + i);
    if (flags && p0 + i < n_pages) flags[row * n_pages + p0 + i] = sel ? 1 : 0;
    bits |= sel ? (1u << i) : 0u;
  }
  if (bitmap) {
    // the selection as bitmap words (bit b of word w: page 32 w + b); with
    // 16 pages a thread, word w is the even thread 2 w's bits and its
    // neighbour's
    static_assert(KPT == 16 || KPT == 32, "one or two threads per bitmap word");
    const int64_t words = (n_pages + 31) / 32;
    int64_t wd = tid;
    if constexpr (KPT == 16) {
      const uint32_t hi = __shfl_xor(bits, 1, 64);
      bits |= hi << 16;
      wd = tid >> 1;
    }
    if ((KPT == 32 || (tid & 1) == 0) && wd < words) bitmap[row * words + wd] = bits;
  }
}

}  // namespace

hipError_t launch_page_meta(const void* k, int64_t kv_st, int64_t kv_sh, int64_t n_kv, int hkv,
                            int d, int page_size, fb_dtype dt, void* kmin, void* kmax,
                            int64_t p_begin, int64_t p_end, int64_t page_cap, hipStream_t s) {
  if (p_end <= p_begin) return hipSuccess;
  const int64_t n_pg = p_end - p_begin;
  const int gpr = d * (dt == FB_BF16 ? 2 : 4) / 16;
  dim3 grid(static_cast<unsigned>((n_pg * gpr + 255) / 256), hkv);
  if (dt == FB_BF16)
    hipLaunchKernelGGL(page_meta_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(k), kv_st, kv_sh, n_kv, d, page_size, p_begin,
                       n_pg, page_cap, static_cast<uint16_t*>(kmin), static_cast<uint16_t*>(kmax));
  else
    hipLaunchKernelGGL(page_meta_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(k), kv_st, kv_sh, n_kv, d, page_size, p_begin,
                       n_pg, page_cap, static_cast<float*>(kmin), static_cast<float*>(kmax));
  return hipGetLastError();
}

hipError_t launch_page_select(const void* q, int64_t q_st, int64_t q_sh, const void* kmin,
                              const void* kmax, int n_q, int hq, int hkv, int d, int64_t n_pages,
                              int64_t page_cap, int k_pages, fb_dtype dt, const uint8_t* active,
                              double* bound, int32_t* pages, uint32_t* bitmap, hipStream_t s) {
  if (n_pages == 0) return hipSuccess;
  const int G = hq / hkv;
  dim3 grid(static_cast<unsigned>((n_pages + kPagesPerBlock - 1) / kPagesPerBlock), hkv);
  // G-chain kernel: 32 pages x TC tokens per workgroup, TC = 8 (G <= 4) or 4 (G = 8)
#define FB_BOUND_G(TT, GG)                                                                      \
  hipLaunchKernelGGL((page_bound_g_kernel<TT, GG, 8 / ((GG + 3) / 4)>),                         \
                     dim3(grid.x, grid.y, (n_q + 8 / ((GG + 3) / 4) - 1) / (8 / ((GG + 3) / 4))), \
                     dim3(256),                                                                 \
                     8 / ((GG + 3) / 4) * GG * d * 4 +                                          \
                         2 * kPagesPerBlock * bound_row_stride<TT>(d) * sizeof(TT), s,          \
                     static_cast<const TT*>(q), q_st, q_sh, static_cast<const TT*>(kmin),       \
                     static_cast<const TT*>(kmax), n_q, hkv, d, n_pages, page_cap, active, bound)
  if (dt == FB_BF16 && G == 4) FB_BOUND_G(uint16_t, 4);
  else if (dt == FB_BF16 && G == 1) FB_BOUND_G(uint16_t, 1);
  else if (dt == FB_BF16 && G == 2) FB_BOUND_G(uint16_t, 2);
  else if (dt == FB_BF16 && G == 8) FB_BOUND_G(uint16_t, 8);
  else if (dt == FB_F32 && G == 1) FB_BOUND_G(float, 1);
  else if (dt == FB_F32 && G == 2) FB_BOUND_G(float, 2);
  else if (dt == FB_F32 && G == 4) FB_BOUND_G(float, 4);
  else if (dt == FB_F32 && G == 8) FB_BOUND_G(float, 8);
  else {
    const int tc = page_bound_tokens(n_q, G, d);
    if (tc < 1) return hipErrorInvalidValue;
    const size_t smem = (static_cast<size_t>(tc) * G * d + 2 * kPagesPerBlock * (d + 1)) * sizeof(float);
    const dim3 gz(grid.x, grid.y, static_cast<unsigned>((n_q + tc - 1) / tc));
    if (dt == FB_BF16)
      hipLaunchKernelGGL(page_bound_kernel<uint16_t>, gz, dim3(256), smem, s,
                         static_cast<const uint16_t*>(q), q_st, q_sh,
                         static_cast<const uint16_t*>(kmin), static_cast<const uint16_t*>(kmax),
                         n_q, tc, hq, hkv, d, n_pages, page_cap, active, bound);
    else
      hipLaunchKernelGGL(page_bound_kernel<float>, gz, dim3(256), smem, s,
                         static_cast<const float*>(q), q_st, q_sh, static_cast<const float*>(kmin),
                         static_cast<const float*>(kmax), n_q, tc, hq, hkv, d, n_pages, page_cap,
                         active, bound);
  }
#undef FB_BOUND_G
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || k_pages <= 0) return e;
  return launch_topk_rows(bound, n_q, hkv, n_pages, k_pages, active, pages, nullptr, bitmap, s);
}

// Tokens per workgroup of the generic bound kernel: as many as keep their
// query rows and the page block's rows within 64 KB of LDS (0: not even one).
int page_bound_tokens(int n_q, int G, int d) {
  const int64_t room = 64 * 1024 / static_cast<int64_t>(sizeof(float)) - 2 * kPagesPerBlock * (d + 1);
  const int64_t per = static_cast<int64_t>(G) * d;
  int64_t tc = room > 0 ? room / per : 0;
  if (tc > n_q) tc = n_q;
  return static_cast<int>(tc);
}

int topk_bitmap_max() { return 256 * 32; }

hipError_t launch_topk_rows(const double* keys, int n_rows, int hkv, int64_t n, int k,
                            const uint8_t* row_active, int32_t* out, uint8_t* flags,
                            uint32_t* bitmap, hipStream_t s) {
  if (k <= 0 || n_rows <= 0) return hipSuccess;
  if (bitmap && n > topk_bitmap_max()) return hipErrorInvalidValue;
  if (n <= 256 * 16)
    hipLaunchKernelGGL(page_topk_reg_kernel<16>, dim3(n_rows, hkv), dim3(256), 0, s, keys, hkv, n,
                       k, row_active, out, flags, bitmap);
  else if (n <= 256 * 32)
    hipLaunchKernelGGL(page_topk_reg_kernel<32>, dim3(n_rows, hkv), dim3(256), 0, s, keys, hkv, n,
                       k, row_active, out, flags, bitmap);
  else
    hipLaunchKernelGGL(page_topk_kernel, dim3(n_rows, hkv), dim3(256), 0, s, keys, hkv, n, k,
                       row_active, out, flags);
  return hipGetLastError();
}

}  // namespace fb
