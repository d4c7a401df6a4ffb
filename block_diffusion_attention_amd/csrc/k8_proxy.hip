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
//  * p[t][i] = sum_c x[t][c] F[c][i]: blocks of 128 consecutive c, each
//    summed in c order with fused multiply-add (a product of two bf16 or two
//    fp32 values is exact in float64, so each step rounds once), the block
//    sums then added in block order;
//  * sim = dot / sqrt(|p|^2 |c|^2), clamped to [-1, 1], with dot, |p|^2 and
//    |c|^2 summed over i in order; both norms 0 -> 1, one -> 0. A proxy equal
//    to its cache gives dot = |p|^2 = |c|^2 and sqrt(dot^2) = dot exactly in
//    binary floating point, so it scores exactly 1.
//
// The block partials are an fp64 FMA-bound contraction (N x D x r): each
// workgroup takes 32 tokens x r dims of one 128-wide block, staged 32 c at a
// time through LDS as float64 (40 KB: four workgroups per CU) (16-byte global loads, the next stage in
// flight while the current one is computed); each thread keeps 4 tokens x
// r/32 dims of accumulators. The float64 FMA pipe needs several waves per
// SIMD: blocks of 128 give 4 per SIMD at 1024 tokens x 4096, rank 128.
#include "fb_internal.h"

namespace fb {
namespace {

constexpr int kProxyBlock = 128;     // c per summation block
constexpr int kTokTile = 32;         // tokens per workgroup (partials)
constexpr int kCStage = 32;          // c per LDS stage
constexpr int kKeyTok = 2;           // tokens per workgroup (keys)
constexpr int kMaxRank = 128;

template <typename T> __device__ __forceinline__ double ldd(const T* p);
template <> __device__ __forceinline__ double ldd<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ double ldd<uint16_t>(const uint16_t* p) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*p) << 16));
}

typedef __attribute__((__vector_size__(2 * sizeof(double)))) double f64x2;

// Element groups of 16 bytes (8 bf16 or 4 fp32) as float64, zeros at and
// past `end`; `vec` = the group is 16-byte aligned (a single load).
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

template <typename T> __device__ __forceinline__ double grp_elem(u32x4v g, int e);
template <> __device__ __forceinline__ double grp_elem<uint16_t>(u32x4v g, int e) {
  const uint32_t w = g[e >> 1];
  return static_cast<double>(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)));
}
template <> __device__ __forceinline__ double grp_elem<float>(u32x4v g, int e) {
  return static_cast<double>(__uint_as_float(g[e]));
}

// The dim held in accumulator slot j of lane ig: pairs 64 q + 2 ig,
// 64 q + 2 ig + 1 (j = 2 q, 2 q + 1) and, for odd OI, 64 (OI / 2) + ig, so
// the lanes of a wave read one contiguous run of LDS per load.
template <int OI>
__device__ __forceinline__ int dim_of(int j, int ig) {
  return (j + 1 < OI || (OI % 2) == 0) ? 32 * (j & ~1) + 2 * ig + (j & 1) : 32 * j + ig;
}

// part[b][t][i] = sum over c in block b, in order, of x[t][c] F[c][i].
// Workgroup: 32 tokens x R dims (R = 32 OI) of one block, 256 threads;
// thread (tg, ig): tokens 4 tg .. 4 tg + 3, the OI dims dim_of(j, ig).
// Each 32-c stage is loaded into registers (16-byte groups) while the
// previous one is computed, then converted into the LDS tiles.
template <typename T, int OI>
__global__ __launch_bounds__(256) void proxy_partials_kernel(const T* x, int64_t x_st,
                                                             const T* f, int n_tok, int d_model,
                                                             int x_vec, double* part) {
  constexpr int R = 32 * OI;
  constexpr int NE = Grp<T>::N;
  constexpr int XGN = kTokTile * kCStage / NE;        // x groups per stage
  constexpr int FGN = kCStage * R / NE;               // F groups per stage
  constexpr int XG = (XGN + 255) / 256;               // per thread
  constexpr int FG = (FGN + 255) / 256;
  __shared__ __attribute__((aligned(16))) double xs[kCStage][kTokTile];   // [c][t]
  __shared__ __attribute__((aligned(16))) double fs[kCStage][R];          // [c][i]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTokTile;
  const int b = blockIdx.y;
  const int c_begin = b * kProxyBlock;
  const int c_end = c_begin + kProxyBlock < d_model ? c_begin + kProxyBlock : d_model;
  const int tg = tid >> 5, ig = tid & 31;
  double acc[4][OI];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < OI; ++j) acc[a][j] = 0.0;

  u32x4v xr[XG], fr[FG];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int v = tid + 256 * k;                 // group v: token v / (64 / NE), c-group v % ...
      const int t = v / (kCStage / NE), c = c0 + (v % (kCStage / NE)) * NE;
      const int tt = t0 + t;
      xr[k] = (v < XGN && tt < n_tok)
                  ? load_grp<T>(x + static_cast<int64_t>(tt) * x_st, c, c_end, x_vec != 0)
                  : u32x4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < FG; ++k) {
      const int v = tid + 256 * k;                 // group v: row v / (R / NE), i-group ...
      const int c = c0 + v / (R / NE), i = (v % (R / NE)) * NE;
      fr[k] = (v < FGN && c < c_end)
                  ? *reinterpret_cast<const u32x4v*>(f + static_cast<int64_t>(c) * R + i)
                  : u32x4v{0u, 0u, 0u, 0u};
    }
  };
  fetch(c_begin);
  for (int c0 = c_begin; c0 < c_end; c0 += kCStage) {
    // the staged groups into LDS as float64 (zeros past the block end or the
    // tokens: a zero product leaves a sum that is not -0 unchanged)
#pragma unroll
    for (int k = 0; k < XG; ++k) {
      const int v = tid + 256 * k;
      const int t = v / (kCStage / NE), c = (v % (kCStage / NE)) * NE;
      if (v < XGN) {
#pragma unroll
        for (int e = 0; e < NE; ++e) xs[c + e][t] = grp_elem<T>(xr[k], e);
      }
    }
#pragma unroll
    for (int k = 0; k < FG; ++k) {
      const int v = tid + 256 * k;
      const int c = v / (R / NE), i = (v % (R / NE)) * NE;
      if (v < FGN) {
#pragma unroll
        for (int e = 0; e < NE; e += 2) {
          const f64x2 w = {grp_elem<T>(fr[k], e), grp_elem<T>(fr[k], e + 1)};
          *reinterpret_cast<f64x2*>(&fs[c][i + e]) = w;
        }
      }
    }
    __syncthreads();
    if (c0 + kCStage < c_end) fetch(c0 + kCStage);
#pragma unroll 4
    for (int c = 0; c < kCStage; ++c) {
      const f64x2 xa = *reinterpret_cast<const f64x2*>(&xs[c][4 * tg]);
      const f64x2 xb = *reinterpret_cast<const f64x2*>(&xs[c][4 * tg + 2]);
      const double xv[4] = {xa[0], xa[1], xb[0], xb[1]};
      double fv[OI];
#pragma unroll
      for (int j = 0; j < OI; j += 2) {
        if (j + 1 < OI) {
          const f64x2 fp = *reinterpret_cast<const f64x2*>(&fs[c][32 * j + 2 * ig]);
          fv[j] = fp[0];
          fv[j + 1] = fp[1];
        } else {
          fv[j] = fs[c][32 * j + ig];
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < OI; ++j) acc[a][j] = __builtin_fma(xv[a], fv[j], acc[a][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + 4 * tg + a;
    if (t >= n_tok) continue;
    double* o = part + (static_cast<int64_t>(b) * n_tok + t) * R;
#pragma unroll
    for (int j = 0; j < OI; ++j) o[dim_of<OI>(j, ig)] = acc[a][j];
  }
}

// Proxies from the block partials (block order), then either the cache fill
// (init) or the cosine similarities against the cache.
__global__ __launch_bounds__(256) void proxy_keys_kernel(const double* part, int n_blocks,
                                                         int n_tok, int rank, int init,
                                                         double* cache, double* proxy,
                                                         double* sim, double* neg_key,
                                                         uint8_t* mask) {
#pragma clang fp contract(off)
  __shared__ double ps[kKeyTok * (kMaxRank + 1)];  // [kKeyTok][rank + 1]
  __shared__ double cs[kKeyTok * (kMaxRank + 1)];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kKeyTok;
  const int rs = rank + 1;
  for (int e = tid; e < kKeyTok * rank; e += 256) {
    const int tl = e / rank, i = e % rank, t = t0 + tl;
    if (t >= n_tok) continue;
    double acc = 0.0;
    for (int b = 0; b < n_blocks; ++b) acc = acc + part[(static_cast<int64_t>(b) * n_tok + t) * rank + i];
    const int64_t o = static_cast<int64_t>(t) * rank + i;
    proxy[o] = acc;
    if (init) {
      cache[o] = acc;
    } else {
      ps[tl * rs + i] = acc;
      cs[tl * rs + i] = cache[o];
    }
  }
  if (init) {
    for (int tl = tid; tl < kKeyTok; tl += 256)
      if (t0 + tl < n_tok) mask[t0 + tl] = 1;
    return;
  }
  __syncthreads();
  if (tid < kKeyTok && t0 + tid < n_tok) {
    const double* p = ps + tid * rs;
    const double* c = cs + tid * rs;
    double dot = 0.0, pp = 0.0, cc = 0.0;
    for (int i = 0; i < rank; ++i) {
      const double a = p[i], q = c[i];
      const double m1 = a * q, m2 = a * a, m3 = q * q;
      dot = dot + m1;
      pp = pp + m2;
      cc = cc + m3;
    }
    double k;
    if (pp == 0.0 || cc == 0.0) {
      k = (pp == 0.0 && cc == 0.0) ? 1.0 : 0.0;
    } else {
      const double den = pp * cc;
      k = dot / __builtin_sqrt(den);
      k = k > 1.0 ? 1.0 : (k < -1.0 ? -1.0 : k);
    }
    const int t = t0 + tid;
    if (sim) sim[t] = k;
    neg_key[t] = -k;
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
  hipLaunchKernelGGL((proxy_partials_kernel<TY, OI>), grid, dim3(256), 0, s,                     \
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
  hipLaunchKernelGGL(proxy_keys_kernel, dim3((n_tok + kKeyTok - 1) / kKeyTok), dim3(256), 0, s,
                     part, n_blocks, n_tok, rank, init, cache, proxy, sim, neg_key, mask);
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
