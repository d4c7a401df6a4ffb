// k8_proxy.hip -- singular-proxy identification of the tokens to recompute.
//
// SPA-Cache (Proxy singolari per la caching adattiva nei modelli linguistici
// diffusivi, technical summary, methodology s1): each token's input state is
// projected onto the rank-r truncated SVD of the value projection (the
// stored factor F = U_r diag(sigma_r), [D, r]), the proxy is compared by
// cosine with the proxy cached for that token, and the least similar tokens
// are recomputed.
//
// Arithmetic (float64; run to run the bits repeat, the order is fixed):
//  * p[t][i] = sum_c x[t][c] F[c][i]: blocks of 512 consecutive c, each
//    the sum of its two halves, each half accumulated 4 c at a time by the
//    float64 matrix instruction (v_mfma_f64_16x16x4f64) in c order (a
//    product of two bf16 or two fp32 values is exact in float64); the block
//    sums then added in block order;
//  * sim = dot / sqrt(|p|^2 |c|^2), clamped to [-1, 1]; dot, |p|^2 and |c|^2
//    each summed in one fixed order (per lane over its dims, then an xor
//    butterfly over the wave); both norms 0 -> 1, one -> 0. A proxy equal to
//    its cache gives dot = |p|^2 = |c|^2 bit for bit and sqrt(dot^2) = dot
//    exactly in binary floating point, so it scores exactly 1.
//
// Launches: the block partials (matrix cores), the proxies and similarities
// (one wave per token), then the selection: rank counting (mask bytes, cache
// rows, selection words) and the ascending id list, or for more than
// kSelMaxTok tokens the radix top-k of the page selector and a scatter.
#include "fb_internal.h"

namespace fb {
namespace {

#ifndef FB_PROXY_BLOCK
#define FB_PROXY_BLOCK 512
#endif
#ifndef FB_PROXY_KSPLIT
#define FB_PROXY_KSPLIT 2
#endif
constexpr int kProxyBlock = FB_PROXY_BLOCK;   // c per summation block
constexpr int kKSplit = FB_PROXY_KSPLIT;      // slices of a block, 4 waves each
constexpr int kTokTile = 32;                  // tokens per workgroup (partials)
constexpr int kCStage = 32;                   // c per LDS stage
constexpr int kMaxRank = 128;

__device__ __forceinline__ double widen(float v) { return v; }
__device__ __forceinline__ double widen(uint16_t v) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(v) << 16));
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Element groups of 16 bytes (8 bf16 or 4 fp32), zeros at and past `end`;
// `vec` = the group is 16-byte aligned (a single load).
template <typename T> struct Grp { static constexpr int N = 16 / sizeof(T); };

template <typename T>
__device__ __forceinline__ u32x4v load_grp(const T* row, int c, int end, bool vec) {
  constexpr int NE = Grp<T>::N;
  if (vec && c + NE <= end) return *reinterpret_cast<const u32x4v*>(row + c);
  u32x4v r = {0u, 0u, 0u, 0u};
  T tmp[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) tmp[e] = c + e < end ? row[c + e] : T(0);
  __builtin_memcpy(&r, tmp, 16);
  return r;
}

// part[b][t][i] = the sum over c in block b of x[t][c] F[c][i]. Workgroup:
// 32 tokens x R dims (R = 32 OI) of one block, kKSplit slices of 4 waves,
// slice h summing the h-th part of the block. In a slice, wave w owns the
// 16 x 16 output tiles w, w + 4, ... (tile q: token half q / (R / 16), dims
// 16 (q % (R / 16)) ..). The operands are staged as stored (bf16 or fp32),
// 32 c at a time, through two LDS buffers per slice, one barrier per stage:
// x tile [t][c] (rows padded by one 16-byte group), F tile [c][i] (rows
// padded by 16 elements), so that the 16 lanes of a quarter-wave read 16
// consecutive tokens (x) or dims (F) of one c, the four quarters four
// consecutive c, on distinct banks; each operand is widened to float64 as it
// is read. The next stage's 16-byte global loads are in flight while the
// current one is computed. At 1024 tokens x 4096, rank 128: 256 workgroups
// of 8 waves, two per SIMD.
template <typename T, int OI>
__global__ __launch_bounds__(256 * kKSplit) void proxy_partials_kernel(
    const T* x, int64_t x_st, const T* f, int n_tok, int d_model, int x_vec, double* part) {
  constexpr int R = 32 * OI;
  constexpr int NE = Grp<T>::N;
  constexpr int XS = kCStage + NE;                    // x row stride (elements)
  constexpr int FS = R + 16;                          // F row stride (elements)
  constexpr int XGN = kTokTile * kCStage / NE;        // x groups per stage
  constexpr int FGN = kCStage * R / NE;               // F groups per stage
  constexpr int XG = (XGN + 255) / 256;               // per thread
  constexpr int FG = (FGN + 255) / 256;
  constexpr int SUB = kProxyBlock / kKSplit;          // c per slice of the block
  __shared__ __attribute__((aligned(16))) T xs[kKSplit][2][kTokTile * XS];
  __shared__ __attribute__((aligned(16))) T fs[kKSplit][2][kCStage * FS];
  const int h = threadIdx.x >> 8;                     // slice
  const int tid = threadIdx.x & 255;
  const int t0 = blockIdx.x * kTokTile;
  const int b = blockIdx.y;
  const int c_begin = b * kProxyBlock;
  const int c_end = c_begin + kProxyBlock < d_model ? c_begin + kProxyBlock : d_model;
  const int s_begin = c_begin + h * SUB;
  const int s_end = s_begin + SUB < c_end ? s_begin + SUB : c_end;
  const int wv = tid >> 6, ln = tid & 63, lr = ln & 15, lk = ln >> 4;
  f64x4 acc[OI];
#pragma unroll
  for (int q = 0; q < OI; ++q) acc[q] = f64x4{0.0, 0.0, 0.0, 0.0};

  u32x4v xr[XG], fr[FG];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int v = tid + 256 * k;
      const int t = v / (kCStage / NE), c = c0 + (v % (kCStage / NE)) * NE;
      const int tt = t0 + t;
      xr[k] = (v < XGN && tt < n_tok)
                  ? load_grp<T>(x + static_cast<int64_t>(tt) * x_st, c, s_end, x_vec != 0)
                  : u32x4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < FG; ++k) {
      const int v = tid + 256 * k;
      const int c = c0 + v / (R / NE), i = (v % (R / NE)) * NE;
      fr[k] = (v < FGN && c < s_end)
                  ? *reinterpret_cast<const u32x4v*>(f + static_cast<int64_t>(c) * R + i)
                  : u32x4v{0u, 0u, 0u, 0u};
    }
  };
  // zeros past the slice end or the tokens: a zero product leaves a sum
  // that is not -0 unchanged
  auto store = [&](int buf) {
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int v = tid + 256 * k;
      const int t = v / (kCStage / NE), c = (v % (kCStage / NE)) * NE;
      if (v < XGN) *reinterpret_cast<u32x4v*>(&xs[h][buf][t * XS + c]) = xr[k];
    }
#pragma unroll
    for (int k = 0; k < FG; ++k) {
      const int v = tid + 256 * k;
      const int c = v / (R / NE), i = (v % (R / NE)) * NE;
      if (v < FGN) *reinterpret_cast<u32x4v*>(&fs[h][buf][c * FS + i]) = fr[k];
    }
  };
  // every slice runs the first slice's stage count (the barriers are shared;
  // a shorter last slice reads zeros)
  const int first_end = c_begin + SUB < c_end ? c_begin + SUB : c_end;
  const int n_st = (first_end - c_begin + kCStage - 1) / kCStage;
  fetch(s_begin);
  store(0);
  __syncthreads();
  if (n_st > 1) fetch(s_begin + kCStage);
  for (int st = 0; st < n_st; ++st) {
    const T* xb = xs[h][st & 1];
    const T* fb = fs[h][st & 1];
#pragma unroll
    for (int c = 0; c < kCStage; c += 4) {
      const double a0 = widen(xb[lr * XS + c + lk]);
      const double a1 = widen(xb[(16 + lr) * XS + c + lk]);
#pragma unroll
      for (int q = 0; q < OI; ++q) {
        const int qi = wv + 4 * q, tt = qi / (R / 16), dt = qi % (R / 16);
        const double bv = widen(fb[(c + lk) * FS + 16 * dt + lr]);
        acc[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(tt ? a1 : a0, bv, acc[q], 0, 0, 0);
      }
    }
    if (st + 1 < n_st) {
      store((st + 1) & 1);
      if (st + 2 < n_st) fetch(s_begin + (st + 2) * kCStage);
      __syncthreads();
    } else {
      // The accumulators are read by vector instructions next. The wait
      // states the compiler put between the last float64 MFMA and such a
      // read have been too few on gfx950 (the last element of a tile read
      // before the MFMA had written it), so wait here: 128 cycles.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile(
          "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\t"
          "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    }
  }
  if constexpr (kKSplit > 1) {
    // the block sum: slice 0's sum plus slice 1's
    __shared__ f64x4 red[4][OI][64];
    if (h == 1) {
#pragma unroll
      for (int q = 0; q < OI; ++q) red[wv][q][ln] = acc[q];
    }
    __syncthreads();
    if (h == 1) return;
#pragma unroll
    for (int q = 0; q < OI; ++q) {
      const f64x4 o = red[wv][q][ln];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[q][r] = acc[q][r] + o[r];
    }
  }
  // lane l holds D[t = l / 16 + 4 r][i = l % 16] of each of its tiles
#pragma unroll
  for (int q = 0; q < OI; ++q) {
    const int qi = wv + 4 * q, tt = qi / (R / 16), dt = qi % (R / 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * tt + lk + 4 * r;
      if (t < n_tok) part[(static_cast<int64_t>(b) * n_tok + t) * R + 16 * dt + lr] = acc[q][r];
    }
  }
}

// Proxies from the block partials (block order), then either the cache fill
// (init) or the cosine similarities against the cache. One wave per token:
// lane l holds dims l and l + 64 (ranks up to 128); dot, |p|^2 and |c|^2 are summed per lane in dim order, then across
// the wave by an xor butterfly (each step adds a lane's value to its
// partner's, so every lane ends with the same bits, and the three sums keep
// one order: a proxy equal to its cache still scores exactly 1).
constexpr int kKeyWaves = 4;          // tokens per workgroup
__global__ __launch_bounds__(256) void proxy_keys_kernel(const double* part, int n_blocks,
                                                         int n_tok, int rank, int init,
                                                         double* cache, double* proxy,
                                                         double* sim, double* neg_key,
                                                         uint8_t* mask) {
#pragma clang fp contract(off)
  const int ln = threadIdx.x & 63;
  const int t = blockIdx.x * kKeyWaves + (threadIdx.x >> 6);
  if (t >= n_tok) return;                          // whole waves; no barrier below
  const bool has0 = ln < rank, has1 = ln + 64 < rank;
  const int64_t bs = static_cast<int64_t>(n_tok) * rank;
  const double* p0 = part + static_cast<int64_t>(t) * rank + ln;
  double s0 = 0.0, s1 = 0.0;
#pragma unroll 8
  for (int b = 0; b < n_blocks; ++b) {
    if (has0) s0 = s0 + p0[b * bs];
    if (has1) s1 = s1 + p0[b * bs + 64];
  }
  const int64_t o = static_cast<int64_t>(t) * rank + ln;
  if (has0) proxy[o] = s0;
  if (has1) proxy[o + 64] = s1;
  if (init) {
    if (has0) cache[o] = s0;
    if (has1) cache[o + 64] = s1;
    if (ln == 0) mask[t] = 1;
    return;
  }
  const double q0 = has0 ? cache[o] : 0.0, q1 = has1 ? cache[o + 64] : 0.0;
  double dot = 0.0, pp = 0.0, cc = 0.0;
  if (has0) {
    const double m1 = s0 * q0, m2 = s0 * s0, m3 = q0 * q0;
    dot = m1;
    pp = m2;
    cc = m3;
  }
  if (has1) {
    const double m1 = s1 * q1, m2 = s1 * s1, m3 = q1 * q1;
    dot = dot + m1;
    pp = pp + m2;
    cc = cc + m3;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    dot = dot + __shfl_xor(dot, m, 64);
    pp = pp + __shfl_xor(pp, m, 64);
    cc = cc + __shfl_xor(cc, m, 64);
  }
  if (ln == 0) {
    double k;
    if (pp == 0.0 || cc == 0.0) {
      k = (pp == 0.0 && cc == 0.0) ? 1.0 : 0.0;
    } else {
      const double den = pp * cc;
      k = dot / __builtin_sqrt(den);
      k = k > 1.0 ? 1.0 : (k < -1.0 ? -1.0 : k);
    }
    if (sim) sim[t] = k;
    neg_key[t] = 0.0 - k;                          // (+0 for both zeros: they tie)
  }
}

// Selection by rank counting, for up to kSelMaxTok tokens. Keys: -sim as
// order-preserving integers (-0 taken as +0); token j's rank is the number of
// keys above its own plus the equal keys of lower ids, so the n_select
// lowest similarities (ties: lower id) are exactly the ranks below n_select.
// Workgroup: 64 tokens (one per lane), 16 waves each counting over a
// sixteenth of the keys (read 64 at a time, one per lane, then broadcast
// lane by lane). The workgroup writes its tokens' mask bytes and its
// selection word (bit l: token 64 blockIdx + l), and copies its selected
// tokens' proxies into the cache. (No workgroup waits on another: the ids
// are listed by the next launch, since an in-kernel hand-over would need
// device-scope fences, each a write-back of the L2 of the fencing XCD.)
constexpr int kSelTok = 64;
constexpr int kSelWaves = 16;
constexpr int kSelMaxTok = 8192;

__device__ __forceinline__ uint64_t sel_key(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  if ((u << 1) == 0) u = 0;                        // -0 -> +0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__global__ __launch_bounds__(1024) void proxy_select_kernel(const double* neg_key, int n_tok,
                                                            int k, const double* proxy, int rank,
                                                            double* cache, uint8_t* mask,
                                                            uint64_t* words) {
  __shared__ uint32_t cnt[kSelWaves][kSelTok];
  __shared__ uint64_t sh_bits;
  const int ln = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = blockIdx.x * kSelTok + ln;
  const uint64_t kj = j < n_tok ? sel_key(neg_key[j]) : 0ull;
  const int per = (n_tok + kSelWaves - 1) / kSelWaves;
  const int i0 = wv * per, i1 = i0 + per < n_tok ? i0 + per : n_tok;
  uint32_t c = 0;
  for (int base = i0; base < i1; base += 64) {
    const int ii = base + ln;
    const uint64_t mine = ii < i1 ? sel_key(neg_key[ii]) : 0ull;
    const uint32_t mlo = static_cast<uint32_t>(mine), mhi = static_cast<uint32_t>(mine >> 32);
    const int m = i1 - base < 64 ? i1 - base : 64;
    const int rel = j - base;                      // keys l < rel have lower ids
    for (int l = 0; l < m; ++l) {
      const uint64_t ki = (static_cast<uint64_t>(__builtin_amdgcn_readlane(mhi, l)) << 32) |
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(mlo, l));
      c += static_cast<uint32_t>((ki > kj) | ((ki == kj) & (l < rel)));
    }
  }
  cnt[wv][ln] = c;
  __syncthreads();
  if (wv == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) r += cnt[w][ln];
    const bool sel = j < n_tok && r < static_cast<uint32_t>(k);
    const uint64_t bits = __ballot(sel);
    if (j < n_tok) mask[j] = sel ? 1 : 0;
    if (ln == 0) {
      sh_bits = bits;
      words[blockIdx.x] = bits;
    }
  }
  __syncthreads();
  // the selected tokens' cache rows: thread (u, i) copies dim i of tokens
  // u, u + 8, ... (all loads issued before the stores)
  const uint64_t bits = sh_bits;
  const int i = threadIdx.x & 127, u = threadIdx.x >> 7;
  double v[kSelTok / 8];
#pragma unroll
  for (int q = 0; q < kSelTok / 8; ++q) {
    const int tl = u + 8 * q;
    const int64_t o = static_cast<int64_t>(blockIdx.x * kSelTok + tl) * rank + i;
    v[q] = (i < rank && ((bits >> tl) & 1ull)) ? proxy[o] : 0.0;
  }
#pragma unroll
  for (int q = 0; q < kSelTok / 8; ++q) {
    const int tl = u + 8 * q;
    const int64_t o = static_cast<int64_t>(blockIdx.x * kSelTok + tl) * rank + i;
    if (i < rank && ((bits >> tl) & 1ull)) cache[o] = v[q];
  }
}

// The selected ids in ascending order from the selection words: one
// workgroup; thread t takes words [t cw, t cw + cw), its first position from
// a block-wide exclusive scan of the words' popcounts.
__global__ __launch_bounds__(1024) void proxy_list_kernel(const uint64_t* words, int n_words,
                                                          int32_t* selected) {
  __shared__ int sh_tot[16];
  const int ln = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int cw = (n_words + 1023) / 1024;
  const int w0 = threadIdx.x * cw;
  int own = 0;
  for (int w = w0; w < w0 + cw && w < n_words; ++w) own += __popcll(words[w]);
  int incl = own;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (ln >= o) incl += v;
  }
  if (ln == 63) sh_tot[wv] = incl;
  __syncthreads();
  int pos = incl - own;
  for (int w = 0; w < wv; ++w) pos += sh_tot[w];
  for (int w = w0; w < w0 + cw && w < n_words; ++w) {
    uint64_t b = words[w];
    while (b) {
      selected[pos++] = w * kSelTok + (__ffsll(static_cast<long long>(b)) - 1);
      b &= b - 1;
    }
  }
}

// The selected tokens' cache rows take their current proxies (the top-k
// wrote the mask).
__global__ __launch_bounds__(128) void proxy_scatter_kernel(const int32_t* selected, int n_tok,
                                                            const double* proxy, int rank,
                                                            double* cache) {
  const int t = selected[blockIdx.x];
  if (t < 0 || t >= n_tok) return;                 // (the top-k emits ids in range)
  const int64_t o = static_cast<int64_t>(t) * rank;
  for (int i = threadIdx.x; i < rank; i += 128) cache[o + i] = proxy[o + i];
}

}  // namespace

bool proxy_rank_ok(int rank) { return rank >= 32 && rank <= kMaxRank && rank % 32 == 0; }

int proxy_n_blocks(int d_model) { return (d_model + kProxyBlock - 1) / kProxyBlock; }

hipError_t launch_proxy_partials(const void* x, int64_t x_st, const void* factor, fb_dtype dt,
                                 int n_tok, int d_model, int rank, double* part, hipStream_t s) {
  const dim3 grid((n_tok + kTokTile - 1) / kTokTile, proxy_n_blocks(d_model));
  // x rows load as 16-byte groups when every row starts 16-byte aligned
  const int esz = dt == FB_BF16 ? 2 : 4;
  const int x_vec = (reinterpret_cast<uintptr_t>(x) % 16 == 0 && (x_st * esz) % 16 == 0) ? 1 : 0;
#define FB_PROXY(TY, OI)                                                                         \
  hipLaunchKernelGGL((proxy_partials_kernel<TY, OI>), grid, dim3(256 * kKSplit), 0, s,              \
                     static_cast<const TY*>(x), x_st, static_cast<const TY*>(factor), n_tok,      \
                     d_model, x_vec, part)
  const int oi = rank / 32;
  if (dt == FB_BF16) {
    if (oi == 1) FB_PROXY(uint16_t, 1);
    else if (oi == 2) FB_PROXY(uint16_t, 2);
    else if (oi == 3) FB_PROXY(uint16_t, 3);
    else FB_PROXY(uint16_t, 4);
  } else {
    if (oi == 1) FB_PROXY(float, 1);
    else if (oi == 2) FB_PROXY(float, 2);
    else if (oi == 3) FB_PROXY(float, 3);
    else FB_PROXY(float, 4);
  }
#undef FB_PROXY
  return hipGetLastError();
}

hipError_t launch_proxy_keys(const double* part, int n_blocks, int n_tok, int rank, int init,
                             double* cache, double* proxy, double* sim, double* neg_key,
                             uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(proxy_keys_kernel, dim3((n_tok + kKeyWaves - 1) / kKeyWaves), dim3(256),
                     0, s, part, n_blocks, n_tok, rank, init, cache, proxy, sim, neg_key, mask);
  return hipGetLastError();
}

int proxy_select_max_tok() { return kSelMaxTok; }

hipError_t launch_proxy_select(const double* neg_key, int n_tok, int n_select,
                               const double* proxy, int rank, double* cache, uint8_t* mask,
                               uint64_t* words, int32_t* selected, hipStream_t s) {
  const int n_words = (n_tok + kSelTok - 1) / kSelTok;
  hipLaunchKernelGGL(proxy_select_kernel, dim3(n_words), dim3(1024), 0, s, neg_key, n_tok,
                     n_select, proxy, rank, cache, mask, words);
  hipLaunchKernelGGL(proxy_list_kernel, dim3(1), dim3(1024), 0, s, words, n_words, selected);
  return hipGetLastError();
}

hipError_t launch_proxy_scatter(const int32_t* selected, int n_select, int n_tok,
                                const double* proxy, int rank, double* cache, hipStream_t s) {
  if (n_select <= 0) return hipSuccess;
  hipLaunchKernelGGL(proxy_scatter_kernel, dim3(n_select), dim3(128), 0, s, selected, n_tok, proxy,
                     rank, cache);
  return hipGetLastError();
}

}  // namespace fb
