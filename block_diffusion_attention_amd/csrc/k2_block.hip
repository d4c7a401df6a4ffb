// k2_block.hip -- the block-internal pass over J_in and the log-space merge
// with the cached block-external pair (FlashBlock technical summary, s2
// "core mechanism", the A_full equation).
//
// Text blocks are small (B <= 16 queries and keys per step): one wave per
// (query head, block query) computes A_in, L_in over the B block keys of its
// KV head (every block query sees every block key), then merges with the
// cached (A_out, L_out) of the same row:
//   m = max(L_out, L_in), w_x = e^{L_x - m},
//   A_full = (w_out A_out + w_in A_in) / (w_out + w_in),
//   L_full = m + ln(w_out + w_in).
// The work is a few hundred KB per step: this pass is bound by launch
// latency, not by bandwidth or MFMA throughput.
#include "fb_internal.h"

#include <math.h>

namespace fb {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <typename T> __device__ __forceinline__ float ld(const T* p);
template <> __device__ __forceinline__ float ld<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void block_small_kernel(BlockParams p) {
  constexpr int NPL = D / 64;
  const int h = blockIdx.x;
  const int t = blockIdx.y;
  const int lane = threadIdx.x;
  const int g = h / p.group;
  __shared__ float qs[D];
  __shared__ float ps[64];

  const T* qrow = static_cast<const T*>(p.q) + static_cast<int64_t>(t) * p.q_st +
                  static_cast<int64_t>(h) * p.q_sh;
  for (int c = lane; c < D; c += 64) qs[c] = ld<T>(qrow + c);
  __syncthreads();

  const T* kb = static_cast<const T*>(p.k) + static_cast<int64_t>(g) * p.k_sh;
  const T* vb = static_cast<const T*>(p.v) + static_cast<int64_t>(g) * p.v_sh;
  float m = kNegInf, l = 0.f, o[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) o[i] = 0.f;

  for (int base = 0; base < p.n_q; base += 64) {
    const int j = base + lane;
    float x = kNegInf;
    if (j < p.n_q) {
      const T* kr = kb + static_cast<int64_t>(j) * p.k_st;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc += qs[c] * ld<T>(kr + c);
      x = acc * p.scale_log2;
    }
    const float mnew = fmaxf(m, wave_max(x));
    const float alpha = exp2f(m - mnew);
    const float pr = exp2f(x - mnew);
    l = l * alpha + wave_sum(pr);
#pragma unroll
    for (int i = 0; i < NPL; ++i) o[i] *= alpha;
    m = mnew;
    ps[lane] = pr;
    __syncthreads();
    const int nb = p.n_q - base < 64 ? p.n_q - base : 64;
    for (int jj = 0; jj < nb; ++jj) {
      const float pj = ps[jj];
      const T* vr = vb + static_cast<int64_t>(base + jj) * p.v_st;
#pragma unroll
      for (int i = 0; i < NPL; ++i) o[i] += pj * ld<T>(vr + lane + 64 * i);
    }
    __syncthreads();
  }

  const int64_t row = static_cast<int64_t>(t) * p.hq + h;
  const float inv = 1.f / l;                       // n_q >= 1, so l >= 1
  const float l_in = (m + log2f(l)) * kLn2;
  const float l_out = p.l_out[row];
  const float mm = fmaxf(l_out, l_in);
  const float w_out = l_out == kNegInf ? 0.f : expf(l_out - mm);
  const float w_in = expf(l_in - mm);
  const float den = w_out + w_in;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    const float a_in = o[i] * inv;
    const float a_out = p.a_out[row * D + c];
    const float a_full = w_out == 0.f ? a_in : (w_out * a_out + w_in * a_in) / den;
    p.a_full[row * D + c] = a_full;
    if (p.a_in) p.a_in[row * D + c] = a_in;
  }
  if (lane == 0) {
    if (p.l_full) p.l_full[row] = mm + logf(den);
    if (p.l_in) p.l_in[row] = l_in;
  }
}

}  // namespace

hipError_t launch_block_small(const BlockParams& p, fb_dtype dt, hipStream_t s) {
  dim3 grid(p.hq, p.n_q);
  if (dt == FB_BF16) {
    if (p.d == 128) hipLaunchKernelGGL((block_small_kernel<uint16_t, 128>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((block_small_kernel<uint16_t, 64>), grid, dim3(64), 0, s, p);
  } else {
    if (p.d == 128) hipLaunchKernelGGL((block_small_kernel<float, 128>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((block_small_kernel<float, 64>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace fb
