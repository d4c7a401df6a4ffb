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

// element e of a 16-byte group of T values, as float
template <typename T> __device__ __forceinline__ float vec_elem(u32x4v w, int e);
template <> __device__ __forceinline__ float vec_elem<float>(u32x4v w, int e) {
  return __uint_as_float(w[e]);
}
template <> __device__ __forceinline__ float vec_elem<uint16_t>(u32x4v w, int e) {
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
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

constexpr int kMaxMergeChunks = 1024;            // the host's split-K chunk limit

// The split-K merge of one row (one wave; lane owns dims lane + 64 i), with
// the operations of the reduce pass in its order: M = the chunks' max L, Mr =
// the cached residual's L (-inf without one), Mall = max(M, Mr); chunk
// weights e^{L_c - Mall} (0 for empty chunks) summed in chunk order (S); per
// dim the weighted partials summed over the first and the second half of
// the chunks, each in chunk order, then added (acc); the residual enters
// with weight e^{L_res - Mr} (Sr, accr) scaled by e^{Mr - Mall}:
// A = (acc + accr w) / (S + Sr w), L = Mall + ln(S + Sr w); A = 0, L = -inf
// when nothing is there.
template <int NPL>
__device__ __forceinline__ void merge_partials(const BlockParams& p, int64_t row, int lane,
                                               float* wts, float (&a)[NPL], float& l) {
  const int nc = p.n_chunks;
  float m = kNegInf;
  for (int ch = lane; ch < nc; ch += 64) m = fmaxf(m, p.part_l[ch * p.rows + row]);
  m = wave_max(m);
  const float l_res = p.res_l ? p.res_l[row] : kNegInf;
  const float mr = l_res;
  const float mall = fmaxf(m, mr);
  for (int ch = lane; ch < nc; ch += 64) {
    const float L = p.part_l[ch * p.rows + row];
    wts[ch] = L == kNegInf ? 0.f : expf(L - mall);
  }
  const float wr = l_res == kNegInf ? 0.f : expf(l_res - mr);
  __syncthreads();
  float S = 0.f;
  for (int ch = 0; ch < nc; ++ch) S += wts[ch];
  const float Sr = p.res_l ? 0.f + wr : 0.f;
  const float wrr = mr != kNegInf ? expf(mr - mall) : 0.f;
  const int64_t cs = p.rows * NPL * 64;            // chunk stride
  const int mid = (nc + 1) / 2;
  const float* pa = p.part_a + row * NPL * 64 + lane;
  // the two halves advance together, 16 chunks each per round, so a round
  // has 2 x 16 x NPL loads in flight; each half still adds in chunk order
  float acc[2][NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) acc[0][i] = acc[1][i] = 0.f;
  auto batch = [&](int hf, int ch) {               // 16 chunks of one half
    float v[16][NPL];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < NPL; ++i) v[u][i] = pa[(ch + u) * cs + 64 * i];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < NPL; ++i) acc[hf][i] += wts[ch + u] * v[u][i];
  };
  int ch0 = 0, ch1 = mid;
  for (; ch0 + 16 <= mid && ch1 + 16 <= nc; ch0 += 16, ch1 += 16) {
    float v0[16][NPL], v1[16][NPL];
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        v0[u][i] = pa[(ch0 + u) * cs + 64 * i];
        v1[u][i] = pa[(ch1 + u) * cs + 64 * i];
      }
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int i = 0; i < NPL; ++i) {
        acc[0][i] += wts[ch0 + u] * v0[u][i];
        acc[1][i] += wts[ch1 + u] * v1[u][i];
      }
  }
  for (; ch0 + 16 <= mid; ch0 += 16) batch(0, ch0);
  for (; ch1 + 16 <= nc; ch1 += 16) batch(1, ch1);
  for (; ch0 < mid; ++ch0)
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc[0][i] += wts[ch0] * pa[ch0 * cs + 64 * i];
  for (; ch1 < nc; ++ch1)
#pragma unroll
    for (int i = 0; i < NPL; ++i) acc[1][i] += wts[ch1] * pa[ch1 * cs + 64 * i];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    float accr = 0.f;
    if (p.res_l) accr += wr * p.res_a[row * NPL * 64 + lane + 64 * i];
    a[i] = mall != kNegInf ? ((acc[0][i] + acc[1][i]) + accr * wrr) / (S + Sr * wrr) : 0.f;
  }
  l = mall != kNegInf ? mall + logf(S + Sr * wrr) : kNegInf;
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
  __shared__ float wts[kMaxMergeChunks];

  if (p.ids_store && h == 0 && t == 0) {
    // the step's decision: taken here (no prefix pass) or by the pass (the
    // previous launch); since-refresh counting keeps the ids of the last
    // recompute step
    const bool reuse = p.decide_on ? text_step_reuse(p.decide, true) : p.mask[0] != 0;
    if (!(p.ids_keep_on_reuse && reuse))
      for (int i = lane; i < p.ids_n; i += 64) p.ids_store[i] = p.ids_cur[i];
  }
  const T* qrow = static_cast<const T*>(p.q) + static_cast<int64_t>(t) * p.q_st +
                  static_cast<int64_t>(h) * p.q_sh;
  const int64_t row = static_cast<int64_t>(t) * p.hq + h;
  const T* kb = static_cast<const T*>(p.k) + static_cast<int64_t>(g) * p.k_sh;
  const T* vb = static_cast<const T*>(p.v) + static_cast<int64_t>(g) * p.v_sh;
  // bf16: the K row of this lane's key among the first 64 and this lane's
  // dims of the first kPreV V rows are loaded before anything else, so a
  // block of up to kPreV tokens needs one memory round trip (with the cached
  // pair and the query row) instead of three
  constexpr bool kPre = sizeof(T) == 2;
  constexpr int kVec = 16 / sizeof(T);
  constexpr int kPreV = 16;
  u32x4v k0[kPre ? D / kVec : 1];
  T v0[kPre ? kPreV : 1][NPL];                     // raw bits, converted where used
  if (kPre) {
    // rows past the block clamp to its last (loaded, never used)
    const int kj = lane < p.n_q ? lane : p.n_q - 1;
    const T* kr = kb + static_cast<int64_t>(kj) * p.k_st;
#pragma unroll
    for (int u = 0; u < D / kVec; ++u) k0[u] = *reinterpret_cast<const u32x4v*>(kr + u * kVec);
#pragma unroll
    for (int jj = 0; jj < kPreV; ++jj) {
      const T* vr = vb + static_cast<int64_t>(jj < p.n_q ? jj : p.n_q - 1) * p.v_st;
#pragma unroll
      for (int i = 0; i < NPL; ++i) v0[jj][i] = vr[lane + 64 * i];
    }
  }
  // the query row (16-byte groups), issued with the prefetch above
  constexpr int kQV = 16 / sizeof(T);
  u32x4v qw = {0u, 0u, 0u, 0u};
  if (lane < D / kQV) qw = *reinterpret_cast<const u32x4v*>(qrow + lane * kQV);
  // the cached pair, loaded with the rest (on a fresh pass it is replaced
  // by the merge of the partials below, and these values go unused)
  float a_out[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) a_out[i] = p.a_out[row * D + lane + 64 * i];
  float l_out = p.l_out[row];
  if (p.part_l && !(p.mask && p.mask[h]) && !(p.active && !p.active[t])) {
    // a fresh prefix pass: merge this row's split-K partials (the same
    // operations in the same order as the reduce pass) into the pair
    merge_partials<NPL>(p, row, lane, wts, a_out, l_out);
    p.cache_l[row] = l_out;                        // (every lane writes the same value)
#pragma unroll
    for (int i = 0; i < NPL; ++i) p.cache_a[row * D + lane + 64 * i] = a_out[i];
  }
  if (lane < D / kQV) {
#pragma unroll
    for (int e = 0; e < kQV; ++e) qs[lane * kQV + e] = vec_elem<T>(qw, e);
    if (p.q_dst)                                   // (after every read of q_dst this step)
      *reinterpret_cast<u32x4v*>(static_cast<T*>(p.q_dst) + row * D + lane * kQV) = qw;
  }
  __syncthreads();

  float m = kNegInf, l = 0.f, o[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) o[i] = 0.f;

  for (int base = 0; base < p.n_q; base += 64) {
    const int j = base + lane;
    float x = kNegInf;
    if (j < p.n_q) {
      // the key row arrives as 16-byte loads issued together (256 bytes a
      // round: one round for a bf16 row of 128), then the dot product runs
      // from registers in dim order
      const T* kr = kb + static_cast<int64_t>(j) * p.k_st;
      constexpr int kR = (256 / sizeof(T)) < D ? 256 / sizeof(T) : D;   // dims per round
      constexpr int kV = 16 / sizeof(T);
      float acc = 0.f;
#pragma unroll
      for (int c0 = 0; c0 < D; c0 += kR) {
        u32x4v kv[kR / kV];
        if (kPre && base == 0) {
#pragma unroll
          for (int u = 0; u < kR / kV; ++u) kv[u] = k0[(c0 / kV + u) % (kPre ? D / kVec : 1)];
        } else {
#pragma unroll
          for (int u = 0; u < kR / kV; ++u) kv[u] = *reinterpret_cast<const u32x4v*>(kr + c0 + u * kV);
        }
#pragma unroll
        for (int u = 0; u < kR / kV; ++u)
#pragma unroll
          for (int e = 0; e < kV; ++e) acc += qs[c0 + u * kV + e] * vec_elem<T>(kv[u], e);
      }
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
    int jj = 0;
    if (kPre && base == 0) {
#pragma unroll
      for (int u = 0; u < kPreV; ++u)
        if (u < nb) {
          const float pj = ps[u];
#pragma unroll
          for (int i = 0; i < NPL; ++i) o[i] += pj * ld<T>(&v0[u % (kPre ? kPreV : 1)][i]);
        }
      jj = nb < kPreV ? nb : kPreV;
    }
    for (; jj < nb; ++jj) {
      const float pj = ps[jj];
      const T* vr = vb + static_cast<int64_t>(base + jj) * p.v_st;
#pragma unroll
      for (int i = 0; i < NPL; ++i) o[i] += pj * ld<T>(vr + lane + 64 * i);
    }
    __syncthreads();
  }

  const float inv = 1.f / l;                       // n_q >= 1, so l >= 1
  const float l_in = (m + log2f(l)) * kLn2;
  const float mm = fmaxf(l_out, l_in);
  const float w_out = l_out == kNegInf ? 0.f : expf(l_out - mm);
  const float w_in = expf(l_in - mm);
  const float den = w_out + w_in;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int c = lane + 64 * i;
    const float a_in = o[i] * inv;
    const float a_full = w_out == 0.f ? a_in : (w_out * a_out[i] + w_in * a_in) / den;
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
