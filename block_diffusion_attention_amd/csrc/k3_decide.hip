// k3_decide.hip -- the reuse controller, on the device, producing integer
// masks that the prefix pass consumes without a host round trip.
//
//  * count     (FlashBlock technical summary, s2 threshold reuse): M = number
//              of block positions whose token id changed; reuse iff M < tau.
//              Changed since the previous step, or (variant) since the ids
//              of the last step that recomputed, which are the ones kept.
//  * head_cos  (same section, per-head selection): cosine of a head's fresh
//              block-external output against its cached one, float64, fixed
//              reduction order; reuse iff sim > gamma. The same pass can copy
//              the fresh pair into the cache for the heads recomputed.
//  * active_mse (LoSA s2, token classification): per-token mean squared
//              query change in float64 with the operations in a fixed order
//              and no fused multiply-add; active iff above the nearest-rank
//              percentile cutoff.
#include "fb_internal.h"

#include <math.h>

namespace fb {
namespace {

__global__ __launch_bounds__(256) void count_kernel(const int32_t* prev, const int32_t* cur, int n,
                                                    int tau, int force, int hq, uint8_t* mask,
                                                    int32_t* m_count, int32_t* store,
                                                    int store_on_recompute) {
  __shared__ int total;
  const int tid = threadIdx.x;
  if (tid == 0) total = 0;
  __syncthreads();
  int c = 0;
  if (prev != nullptr)
    for (int i = tid; i < n; i += blockDim.x) c += prev[i] != cur[i] ? 1 : 0;
  atomicAdd(&total, c);
  __syncthreads();                                 // every read of prev is done
  // prev == NULL: first step of a block, every token is new to the cache.
  // force: -1 decide, 0 recompute, 1 reuse.
  const int M = prev != nullptr ? total : n;
  const bool reuse = force == 1 ? true : (force == 0 ? false : (M < tau));
  for (int h = tid; h < hq; h += blockDim.x) mask[h] = reuse ? 1 : 0;
  if (tid == 0 && m_count) *m_count = M;
  // since-refresh counting keeps the ids of the last compute step
  if (store && !(store_on_recompute && reuse))
    for (int i = tid; i < n; i += blockDim.x) store[i] = cur[i];
}

// Partial sums of <a, b>, |a|^2, |b|^2 for head h over a chunk of rows.
// Every product of two floats is exact in float64; the chunk sum uses a
// fixed tree, the chunk partials are summed in order by the finaliser.
// Per (chunk of rows, head): float64 dot, |x|^2, |y|^2 of the head's rows
// lo .. hi, each thread summing its elements in order, then a fixed tree over
// the threads. vec: 16-byte loads (bases 16-byte aligned, d % 4 == 0), eight
// per array in flight per thread. a_copy (nullable): the probe is also
// written there after it was read (the cache takes the fresh output of a head
// that was recomputed), with l_src -> l_copy for the chunk's rows.
__global__ __launch_bounds__(256) void head_cos_partial_kernel(
    const float* a_cached, const float* a_probe, int n_q, int hq, int d, const uint8_t* mask_in,
    int rows_per_chunk, int vec, double* ws, float* a_copy, const float* l_src, float* l_copy) {
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (mask_in && mask_in[h]) return;
  const int lo = chunk * rows_per_chunk;
  const int hi = lo + rows_per_chunk < n_q ? lo + rows_per_chunk : n_q;
  double dot = 0.0, nx = 0.0, ny = 0.0;
  if (vec) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int kU = 8;
    const int vpr = d / 4;                           // 16-byte groups per row
    const int n_vec = (hi - lo) * vpr;
    for (int v0 = 0; v0 < n_vec; v0 += kU * 256) {
      f32x4 xv[kU], yv[kU];
      int64_t at[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int v = v0 + u * 256 + tid;
        const int t = lo + (v < n_vec ? v / vpr : 0), g = v < n_vec ? v % vpr : 0;
        at[u] = (static_cast<int64_t>(t) * hq + h) * d + 4 * g;
        if (v < n_vec) {
          xv[u] = *reinterpret_cast<const f32x4*>(a_probe + at[u]);
          yv[u] = *reinterpret_cast<const f32x4*>(a_cached + at[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (v0 + u * 256 + tid >= n_vec) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double x = xv[u][e], y = yv[u][e];
          dot += x * y;
          nx += x * x;
          ny += y * y;
        }
        if (a_copy) *reinterpret_cast<f32x4*>(a_copy + at[u]) = xv[u];
      }
    }
  } else {
    const int64_t n_el = static_cast<int64_t>(hi - lo) * d;
    for (int64_t e = tid; e < n_el; e += 256) {
      const int64_t t = lo + e / d, c = e % d;
      const int64_t idx = (t * hq + h) * d + c;
      const double x = a_probe[idx], y = a_cached[idx];
      dot += x * y;
      nx += x * x;
      ny += y * y;
      if (a_copy) a_copy[idx] = a_probe[idx];
    }
  }
  if (l_copy)
    for (int t = lo + tid; t < hi; t += 256) l_copy[t * hq + h] = l_src[t * hq + h];
  __shared__ double red[3][256];
  red[0][tid] = dot;
  red[1][tid] = nx;
  red[2][tid] = ny;
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
      red[2][tid] += red[2][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    double* o = ws + (static_cast<int64_t>(chunk) * hq + h) * 3;
    o[0] = red[0][0];
    o[1] = red[1][0];
    o[2] = red[2][0];
  }
}

// One workgroup: every chunk's (dot, |x|^2, |y|^2) is read into LDS at once
// (one round trip instead of one per chunk), then thread h adds its head's
// in chunk order. sim = dot / sqrt(|x|^2 |y|^2) (a probe equal to its cache
// then scores exactly 1: sqrt(dot^2) = dot), clamped to [-1, 1]; both sides
// zero -> 1, one side zero -> 0.
constexpr int kCosStage = 4096;                  // staged doubles (chunks x heads x 3)

__global__ __launch_bounds__(256) void head_cos_final_kernel(int hq, int n_chunks,
                                                             const uint8_t* mask_in, double gamma,
                                                             const double* ws, double* sim,
                                                             uint8_t* mask) {
  __shared__ double st[kCosStage];
  const int n = n_chunks * hq * 3;
  const bool staged = n <= kCosStage;
  if (staged) {
    for (int i0 = 0; i0 < n; i0 += 8 * 256) {     // eight loads in flight per thread
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256 + static_cast<int>(threadIdx.x);
        v[u] = i < n ? ws[i] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 256 + static_cast<int>(threadIdx.x);
        if (i < n) st[i] = v[u];
      }
    }
  }
  __syncthreads();
  const double* src = staged ? st : ws;
  for (int h = threadIdx.x; h < hq; h += 256) {
    if (mask_in && mask_in[h]) {
      mask[h] = 1;
      continue;
    }
    double dot = 0.0, nx = 0.0, ny = 0.0;
    for (int c = 0; c < n_chunks; ++c) {
      const double* o = src + (static_cast<int64_t>(c) * hq + h) * 3;
      dot += o[0];
      nx += o[1];
      ny += o[2];
    }
    double s;
    if (nx == 0.0 || ny == 0.0) {
      s = (nx == 0.0 && ny == 0.0) ? 1.0 : 0.0;
    } else {
      const double den = nx * ny;
      // (a product past the double range falls back to the two roots)
      s = (den > 0.0 && den < __builtin_huge_val()) ? dot / sqrt(den)
                                                     : dot / (sqrt(nx) * sqrt(ny));
      s = s > 1.0 ? 1.0 : (s < -1.0 ? -1.0 : s);
    }
    sim[h] = s;
    mask[h] = s > gamma ? 1 : 0;
  }
}

template <typename T> __device__ __forceinline__ double ldd(const T* p);
template <> __device__ __forceinline__ double ldd<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ double ldd<uint16_t>(const uint16_t* p) {
  return static_cast<double>(__uint_as_float(static_cast<uint32_t>(*p) << 16));
}

// One workgroup per block token. Thread h adds the squared differences of
// head h in dim order (diff, square, add in float64; contraction into fused
// multiply-add is disabled), and thread 0 adds the per-head sums in head
// order: the same rounding sequence as a scalar loop in that order.
template <typename T>
__global__ __launch_bounds__(256) void active_mse_kernel(const T* q_prev, const T* q_cur, int hq,
                                                         int d, double* mse_out, double* ws) {
#pragma clang fp contract(off)
  __shared__ double part[256];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t per = static_cast<int64_t>(hq) * d;
  const T* a = q_prev + t * per;
  const T* b = q_cur + t * per;
  double total = 0.0;
  for (int h0 = 0; h0 < hq; h0 += 256) {           // 256 heads per pass
    const int h = h0 + tid;
    if (h < hq) {
      const T* ah = a + static_cast<int64_t>(h) * d;
      const T* bh = b + static_cast<int64_t>(h) * d;
      double acc = 0.0;
      for (int j = 0; j < d; ++j) {
        const double diff = ldd<T>(bh + j) - ldd<T>(ah + j);
        const double sq = diff * diff;
        acc = acc + sq;
      }
      part[tid] = acc;
    }
    __syncthreads();
    if (tid == 0) {
      const int n = hq - h0 < 256 ? hq - h0 : 256;
      for (int i = 0; i < n; ++i) total = total + part[i];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double v = total / static_cast<double>(per);
    ws[t] = v;
    if (mse_out) mse_out[t] = v;
  }
}

// Nearest-rank cutoff over the block's MSE values (the rank-th smallest,
// rank = ceil(pct * n / 100)) and the active flags MSE > cutoff.
__global__ __launch_bounds__(256) void active_cut_kernel(int n_q, int pct, const double* ws,
                                                         uint8_t* active) {
  __shared__ double cutoff;
  const int tid = threadIdx.x;
  int rank = (pct * n_q + 99) / 100;
  if (rank < 1) rank = 1;
  for (int t = tid; t < n_q; t += blockDim.x) {
    const double v = ws[t];
    int less = 0, leq = 0;
    for (int u = 0; u < n_q; ++u) {
      const double x = ws[u];
      less += x < v ? 1 : 0;
      leq += x <= v ? 1 : 0;
    }
    if (less < rank && rank <= leq) cutoff = v;    // every writer writes the same value
  }
  __syncthreads();
  const double c = cutoff;
  for (int t = tid; t < n_q; t += blockDim.x) active[t] = ws[t] > c ? 1 : 0;
}

// One sparse denoising step's token bookkeeping in one workgroup (the block
// sizes of text block diffusion): the active set by the same arithmetic as
// active_mse_kernel + active_cut_kernel (mode 1) or a constant (mode 0),
// then q_prev <- q_cur for the next step's comparison.
constexpr int kStepChains = 4096;                  // (token, head) sums held in LDS

template <typename T>
__global__ __launch_bounds__(1024) void active_step_kernel(T* q_prev, const T* q_cur, int64_t q_st,
                                                           int64_t q_sh, int n_q, int hq, int d,
                                                           int mode, uint8_t fill, int pct,
                                                           double* mse_out, uint8_t* active) {
#pragma clang fp contract(off)
  __shared__ double part[kStepChains];
  __shared__ double mse_s[1024];
  __shared__ double cutoff;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int chains = n_q * hq;
  if (mode == 1) {
    // rows are 16-byte aligned: d is 64 or 128 and strides multiples of 8
    for (int i = tid; i < chains; i += nt) {
      const int t = i / hq, h = i % hq;
      part[i] = sq_diff_sum<T>(q_prev + static_cast<int64_t>(i) * d, q_cur + t * q_st + h * q_sh, d);
    }
    __syncthreads();
    for (int t = tid; t < n_q; t += nt) {
      double total = 0.0;
      for (int h = 0; h < hq; ++h) total = total + part[t * hq + h];
      const double v = total / static_cast<double>(hq * d);
      mse_s[t] = v;
      if (mse_out) mse_out[t] = v;
    }
    __syncthreads();
    int rank = (pct * n_q + 99) / 100;
    if (rank < 1) rank = 1;
    for (int t = tid; t < n_q; t += nt) {
      const double v = mse_s[t];
      int less = 0, leq = 0;
      for (int u = 0; u < n_q; ++u) {
        less += mse_s[u] < v ? 1 : 0;
        leq += mse_s[u] <= v ? 1 : 0;
      }
      if (less < rank && rank <= leq) cutoff = v;  // every writer writes the same value
    }
    __syncthreads();
    for (int t = tid; t < n_q; t += nt) active[t] = mse_s[t] > cutoff ? 1 : 0;
  } else {
    for (int t = tid; t < n_q; t += nt) active[t] = fill;
  }
  __syncthreads();                                 // every read of q_prev is done
  // copy as 16-byte vectors, four loads in flight per thread before the stores
  typedef unsigned int u32x4c __attribute__((ext_vector_type(4)));
  constexpr int kVc = 16 / sizeof(T);
  const int vpr = d / kVc;                         // vectors per (token, head) row
  const int n_vec = chains * vpr;
  for (int v0 = 0; v0 < n_vec; v0 += 4 * nt) {
    u32x4c x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * nt + tid;
      if (v < n_vec) {
        const int i = v / vpr, j = v % vpr;
        const int t = i / hq, h = i % hq;
        x[u] = *reinterpret_cast<const u32x4c*>(q_cur + t * q_st + h * q_sh + j * kVc);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + u * nt + tid;
      if (v < n_vec) *reinterpret_cast<u32x4c*>(q_prev + static_cast<int64_t>(v) * kVc) = x[u];
    }
  }
}

__global__ __launch_bounds__(256) void fill_u8_kernel(uint8_t* p, int n, uint8_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

template <typename T>
__global__ __launch_bounds__(256) void copy_rows_kernel(const T* src, int64_t st, int64_t sh, T* dst,
                                                        int n_q, int hq, int d) {
  const int64_t n_el = static_cast<int64_t>(n_q) * hq * d;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n_el;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / (static_cast<int64_t>(hq) * d), h = (e / d) % hq, c = e % d;
    dst[e] = src[t * st + h * sh + c];
  }
}

}  // namespace

hipError_t launch_fill_u8(uint8_t* p, int n, uint8_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u8_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, int64_t st, int64_t sh, void* dst, int n_q, int hq,
                            int d, fb_dtype dt, hipStream_t s) {
  const int64_t n_el = static_cast<int64_t>(n_q) * hq * d;
  int nb = static_cast<int>((n_el + 255) / 256);
  if (nb > 2048) nb = 2048;
  if (dt == FB_BF16)
    hipLaunchKernelGGL(copy_rows_kernel<uint16_t>, dim3(nb), dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), st, sh, static_cast<uint16_t*>(dst), n_q,
                       hq, d);
  else
    hipLaunchKernelGGL(copy_rows_kernel<float>, dim3(nb), dim3(256), 0, s,
                       static_cast<const float*>(src), st, sh, static_cast<float*>(dst), n_q, hq, d);
  return hipGetLastError();
}

hipError_t launch_count(const int32_t* ids_prev, const int32_t* ids_cur, int n_q, int tau,
                        int force, int hq, uint8_t* mask, int32_t* m_count, int32_t* ids_store,
                        int store_on_recompute, hipStream_t s) {
  hipLaunchKernelGGL(count_kernel, dim3(1), dim3(256), 0, s, ids_prev, ids_cur, n_q, tau, force, hq,
                     mask, m_count, ids_store, store_on_recompute);
  return hipGetLastError();
}

int head_cos_chunks(int n_q) {
  const int rows_per_chunk = 64;
  return (n_q + rows_per_chunk - 1) / rows_per_chunk;
}

hipError_t launch_head_cos(const float* a_cached, const float* a_probe, int n_q, int hq, int d,
                           const uint8_t* mask_in, double gamma, double* sim, uint8_t* mask,
                           double* ws, int n_chunks, float* a_copy, const float* l_src,
                           float* l_copy, hipStream_t s) {
  const int rows_per_chunk = 64;
  const auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const int vec = (d % 4 == 0 && al16(a_cached) && al16(a_probe) && (!a_copy || al16(a_copy)))
                      ? 1 : 0;
  hipLaunchKernelGGL(head_cos_partial_kernel, dim3(n_chunks, hq), dim3(256), 0, s, a_cached,
                     a_probe, n_q, hq, d, mask_in, rows_per_chunk, vec, ws, a_copy, l_src, l_copy);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_cos_final_kernel, dim3(1), dim3(256), 0, s, hq, n_chunks, mask_in, gamma,
                     ws, sim, mask);
  return hipGetLastError();
}

hipError_t launch_active_mse(const void* q_prev, const void* q_cur, fb_dtype dt, int n_q, int hq,
                             int d, int pct, double* mse, uint8_t* active, double* ws,
                             hipStream_t s) {
  if (n_q < 1) return hipSuccess;
  if (dt == FB_BF16)
    hipLaunchKernelGGL(active_mse_kernel<uint16_t>, dim3(n_q), dim3(256), 0, s,
                       static_cast<const uint16_t*>(q_prev), static_cast<const uint16_t*>(q_cur),
                       hq, d, mse, ws);
  else
    hipLaunchKernelGGL(active_mse_kernel<float>, dim3(n_q), dim3(256), 0, s,
                       static_cast<const float*>(q_prev), static_cast<const float*>(q_cur), hq, d,
                       mse, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(active_cut_kernel, dim3(1), dim3(256), 0, s, n_q, pct, ws, active);
  return hipGetLastError();
}

bool active_step_fits(int n_q, int hq) {
  return n_q >= 1 && n_q <= 1024 && static_cast<int64_t>(n_q) * hq <= kStepChains;
}

hipError_t launch_active_step(void* q_prev, const void* q_cur, int64_t q_st, int64_t q_sh,
                              fb_dtype dt, int n_q, int hq, int d, int mode, uint8_t fill, int pct,
                              double* mse, uint8_t* active, hipStream_t s) {
  if (dt == FB_BF16)
    hipLaunchKernelGGL(active_step_kernel<uint16_t>, dim3(1), dim3(1024), 0, s,
                       static_cast<uint16_t*>(q_prev), static_cast<const uint16_t*>(q_cur), q_st,
                       q_sh, n_q, hq, d, mode, fill, pct, mse, active);
  else
    hipLaunchKernelGGL(active_step_kernel<float>, dim3(1), dim3(1024), 0, s,
                       static_cast<float*>(q_prev), static_cast<const float*>(q_cur), q_st, q_sh,
                       n_q, hq, d, mode, fill, pct, mse, active);
  return hipGetLastError();
}


}  // namespace fb
