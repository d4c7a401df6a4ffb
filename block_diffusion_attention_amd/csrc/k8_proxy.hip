// k8_proxy.hip -- singular-proxy identification of the tokens to recompute.
//
// SPA-Cache (Proxy singolari per la caching adattiva nei modelli linguistici
// diffusivi, technical summary, methodology s1): each token's input state is
// projected onto the rank-r truncated SVD of the value projection (the
// stored factor F = U_r diag(sigma_r), [D, r]), the proxy is compared by
// cosine with the proxy cached for that token, and the least similar tokens
// are recomputed.
//
// Arithmetic, fixed so that every bit is reproducible:
//  * p[t][i] = sum_c x[t][c] F[c][i] in float64, in blocks of 512
//    consecutive c: each block summed in c order with fused multiply-add
//    (a product of two bf16 or two fp32 values is exact in float64, so each
//    step rounds once, as a multiply followed by an add would), the block
//    sums then added in block order;
//  * key = sign(cos) cos^2 = dot^2 / (|p|^2 |c|^2), negated when dot < 0
//    (and the quotient is not 0), with dot, |p|^2 and |c|^2 summed over i in
//    order from separately rounded products; both norms 0 -> 1, one -> 0.
//
// The block partials are an fp64 FMA-bound contraction (N x D x r): each
// workgroup takes 32 tokens x r dims of one 512-wide block, staged 64 c at a
// time through LDS as float64; each thread keeps 4 tokens x r/32 dims of
// accumulators and reads its operands with 16-byte LDS loads.
#include "fb_internal.h"

namespace fb {
namespace {

constexpr int kProxyBlock = 512;     // c per summation block
constexpr int kTokTile = 32;         // tokens per workgroup (partials)
constexpr int kCStage = 64;          // c per LDS stage
constexpr int kKeyTok = 32;          // tokens per workgroup (keys)
constexpr int kMaxRank = 128;

template <typename T> __device__ __forceinline__ double ldd(const T* p);
template <> __device__ __forceinline__ double ldd<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ double ldd<uint16_t>(const uint16_t* p) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*p) << 16));
}

typedef __attribute__((__vector_size__(2 * sizeof(double)))) double f64x2;

// part[b][t][i] = sum over c in block b, in order, of x[t][c] F[c][i].
// Thread (tg, ig): tokens 4 tg .. 4 tg + 3, dims OI ig .. OI ig + OI - 1.
template <typename T, int OI>
__global__ __launch_bounds__(256) void proxy_partials_kernel(const T* x, int64_t x_st,
                                                             const T* f, int n_tok, int d_model,
                                                             double* part) {
  constexpr int R = 32 * OI;
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

  for (int c0 = c_begin; c0 < c_end; c0 += kCStage) {
    // stage x[t0 .. t0 + 31][c0 .. c0 + 63] and F[c0 .. c0 + 63][0 .. R);
    // positions past the block, the width or the tokens read as zero (a
    // zero product leaves a sum that is not -0 unchanged)
    for (int e = tid; e < kCStage * kTokTile; e += 256) {
      const int t = e / kCStage, c = e % kCStage;          // consecutive threads: consecutive c
      const int tt = t0 + t, cc = c0 + c;
      xs[c][t] = (tt < n_tok && cc < c_end) ? ldd<T>(x + static_cast<int64_t>(tt) * x_st + cc) : 0.0;
    }
    for (int e = tid; e < kCStage * R; e += 256) {
      const int c = e / R, i = e % R;
      const int cc = c0 + c;
      fs[c][i] = cc < c_end ? ldd<T>(f + static_cast<int64_t>(cc) * R + i) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kCStage; ++c) {
      const f64x2 xa = *reinterpret_cast<const f64x2*>(&xs[c][4 * tg]);
      const f64x2 xb = *reinterpret_cast<const f64x2*>(&xs[c][4 * tg + 2]);
      const double xv[4] = {xa[0], xa[1], xb[0], xb[1]};
      double fv[OI];
#pragma unroll
      for (int j = 0; j < OI; j += 2) {
        if (j + 1 < OI) {
          const f64x2 fp = *reinterpret_cast<const f64x2*>(&fs[c][OI * ig + j]);
          fv[j] = fp[0];
          fv[j + 1] = fp[1];
        } else {
          fv[j] = fs[c][OI * ig + j];
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
    double* o = part + (static_cast<int64_t>(b) * n_tok + t) * R + OI * ig;
#pragma unroll
    for (int j = 0; j < OI; ++j) o[j] = acc[a][j];
  }
}

// Proxies from the block partials (block order), then either the cache fill
// (init) or the ranking keys against the cache.
__global__ __launch_bounds__(256) void proxy_keys_kernel(const double* part, int n_blocks,
                                                         int n_tok, int rank, int init,
                                                         double* cache, double* proxy,
                                                         double* key, double* neg_key,
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
    const double den = pp * cc;
    double k;
    if (den == 0.0) {
      k = (pp == 0.0 && cc == 0.0) ? 1.0 : 0.0;
    } else {
      const double d2 = dot * dot;
      const double q = d2 / den;
      k = (dot < 0.0 && q != 0.0) ? -q : q;
    }
    const int t = t0 + tid;
    if (key) key[t] = k;
    neg_key[t] = -k;
  }
}

// The selected tokens: mask 1 and the cache takes their current proxies.
__global__ __launch_bounds__(128) void proxy_scatter_kernel(const int32_t* selected, int n_tok,
                                                            const double* proxy, int rank,
                                                            double* cache, uint8_t* mask) {
  const int t = selected[blockIdx.x];
  if (t < 0 || t >= n_tok) return;                 // (the top-k emits ids in range)
  if (threadIdx.x == 0) mask[t] = 1;
  const int64_t o = static_cast<int64_t>(t) * rank;
  for (int i = threadIdx.x; i < rank; i += 128) cache[o + i] = proxy[o + i];
}

}  // namespace

bool proxy_rank_ok(int rank) { return rank >= 32 && rank <= kMaxRank && rank % 32 == 0; }

int proxy_n_blocks(int d_model) { return (d_model + kProxyBlock - 1) / kProxyBlock; }

hipError_t launch_proxy_partials(const void* x, int64_t x_st, const void* factor, fb_dtype dt,
                                 int n_tok, int d_model, int rank, double* part, hipStream_t s) {
  const dim3 grid((n_tok + kTokTile - 1) / kTokTile, proxy_n_blocks(d_model));
#define FB_PROXY(TT, OI)                                                                         \
  hipLaunchKernelGGL((proxy_partials_kernel<TT, OI>), grid, dim3(256), 0, s,                     \
                     static_cast<const TT*>(x), x_st, static_cast<const TT*>(factor), n_tok,      \
                     d_model, part)
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
                             double* cache, double* proxy, double* key, double* neg_key,
                             uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(proxy_keys_kernel, dim3((n_tok + kKeyTok - 1) / kKeyTok), dim3(256), 0, s,
                     part, n_blocks, n_tok, rank, init, cache, proxy, key, neg_key, mask);
  return hipGetLastError();
}

hipError_t launch_proxy_scatter(const int32_t* selected, int n_select, int n_tok,
                                const double* proxy, int rank, double* cache, uint8_t* mask,
                                hipStream_t s) {
  if (n_select <= 0) return hipSuccess;
  hipLaunchKernelGGL(proxy_scatter_kernel, dim3(n_select), dim3(128), 0, s, selected, n_tok, proxy,
                     rank, cache, mask);
  return hipGetLastError();
}

}  // namespace fb
