// probe_stream.hip -- probes for the benchmark's rooflines: the achievable
// HBM read rate on this part, from a read-only streaming kernel over two
// buffers (the prefix K and V the attention pass reads) with the same access
// style as that pass (16-byte non-temporal loads, several in flight per
// lane) and no arithmetic beyond an XOR that keeps the loads live; the
// float64 and bf16 matrix-core rates (independent MFMA chains, nothing
// else); the launch floor. Not part of the FlashBlock ABI: built as its own library,
// used by the benchmark only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;           // 16-byte loads in flight per lane
constexpr int64_t kChunk = int64_t(kThreads) * kUnroll * 16;   // bytes per round of a workgroup

// Workgroup w reads rounds w, w + grid, w + 2 grid, ... of the concatenation
// of a and b (each a multiple of 16 bytes); bytes past a's end come from b.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* a, int64_t a_vecs,
                                                               const u32x4* b, int64_t b_vecs,
                                                               uint32_t* out) {
  const int64_t total = a_vecs + b_vecs;
  const int64_t per_round = kChunk / 16;
  uint32_t acc = 0;
  for (int64_t r = blockIdx.x; r * per_round < total; r += gridDim.x) {
    const int64_t base = r * per_round + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + int64_t(u) * kThreads;
      if (i < a_vecs) {
        v[u] = __builtin_nontemporal_load(a + i);
      } else if (i < total) {
        v[u] = __builtin_nontemporal_load(b + (i - a_vecs));
      } else {
        v[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per workgroup: thread 0's value (the XOR of the rest is folded
  // through a shuffle so no load is dead)
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t wave_acc[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int w = 0; w < kThreads / 64; ++w) x ^= wave_acc[w];
    out[blockIdx.x] = x;
  }
}

__global__ void empty_kernel() {}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// The float64 matrix-core rate: each wave runs 4 independent accumulator
// chains of v_mfma_f64_16x16x4f64 (2048 flops each) for `iters` rounds; the
// lane's sum goes to out so that nothing is dead.
__global__ __launch_bounds__(256) void f64_mfma_kernel(double* out, int iters) {
  const int l = threadIdx.x & 63;
  const double a = 1.0 + l * 1e-3, b = 1.0 - l * 1e-3;
  f64x4 c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) c[q] = f64x4{0.0, 0.0, 0.0, 0.0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c[q], 0, 0, 0);
  }
  // explicit wait before vector reads of the accumulators (128 cycles)
  __builtin_amdgcn_sched_barrier(0);
  asm volatile(
      "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15\n\t"
      "s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += c[q][0] + c[q][1] + c[q][2] + c[q][3];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// The bf16 matrix-core rate: each wave runs 4 independent accumulator chains
// of v_mfma_f32_32x32x16_bf16 (32,768 flops each), consecutive MFMAs going to
// different accumulators, for `iters` rounds; the lane's sum goes to out.
__global__ __launch_bounds__(256) void bf16_mfma_kernel(float* out, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = static_cast<__bf16>(1.0f + 1e-3f * (l + i));
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) b[q][i] = static_cast<__bf16>(1.0f - 1e-3f * (l + i + q));
  f32x16 c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) c[q] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        c[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[kk], c[q], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[q][i];
  out[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// n_workgroups workgroups of 256 threads (4 waves) of the bf16 MFMA rate
// kernel, 16 MFMAs per wave per round for `iters` rounds: 524,288 * iters
// flops per wave. out: device [n_workgroups * 256] float32. Returns 0 on
// success, 1 on invalid arguments, 2 on a launch error.
int fb_probe_bf16_mfma(int n_workgroups, int iters, float* out, hipStream_t stream) {
  if (n_workgroups < 1 || iters < 1 || !out) return 1;
  hipLaunchKernelGGL(bf16_mfma_kernel, dim3(n_workgroups), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// n_workgroups workgroups of 256 threads (4 waves) of the float64 MFMA rate
// kernel, 4 MFMAs per wave per round for `iters` rounds: 8192 * iters flops
// per wave. out: device [n_workgroups * 256] float64. Returns 0 on
// success, 1 on invalid arguments, 2 on a launch error.
int fb_probe_f64_mfma(int n_workgroups, int iters, double* out, hipStream_t stream) {
  if (n_workgroups < 1 || iters < 1 || !out) return 1;
  hipLaunchKernelGGL(f64_mfma_kernel, dim3(n_workgroups), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// n back-to-back launches of an empty one-wave kernel on `stream`: the
// launch floor a sequence of n dependent kernels cannot go below.
int fb_probe_empty_launches(int n, hipStream_t stream) {
  if (n < 0) return 1;
  for (int i = 0; i < n; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Reads a_bytes at a and b_bytes at b (device, 16-byte aligned, sizes
// multiples of 16) once; out: device [n_workgroups] uint32 (one word each).
// Returns 0 on success, 1 on invalid arguments, 2 on a launch error.
int fb_probe_stream_read(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes,
                         uint32_t* out, int n_workgroups, hipStream_t stream) {
  if (a_bytes < 0 || b_bytes < 0 || (a_bytes % 16) != 0 || (b_bytes % 16) != 0) return 1;
  if ((a_bytes > 0 && !a) || (b_bytes > 0 && !b) || !out || n_workgroups < 1) return 1;
  if ((reinterpret_cast<uintptr_t>(a) % 16) != 0 || (reinterpret_cast<uintptr_t>(b) % 16) != 0)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(n_workgroups), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(a), a_bytes / 16, static_cast<const u32x4*>(b),
                     b_bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
