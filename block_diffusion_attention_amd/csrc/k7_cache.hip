// k7_cache.hip -- a finished block joins the prefix KV cache.
//
// FlashBlock technical summary, s1 problem statement: block-wise decoding
// keeps a KV cache that grows as blocks finish, and every denoising step of
// the next block attends over all of it (J_out of s2 "core mechanism").
// Appending is a strided copy of the block's B x Hkv rows of K and V into the
// cache storage after its last token; each row is d elements, a multiple of
// 16 bytes, moved as 16-byte words (one per lane, rows contiguous across
// lanes, so each wave instruction covers whole rows).
#include "fb_internal.h"

namespace fb {
namespace {

__global__ __launch_bounds__(256) void kv_append_kernel(const char* k_src, int64_t ks_t,
                                                        int64_t ks_h, const char* v_src,
                                                        int64_t vs_t, int64_t vs_h, char* k_dst,
                                                        char* v_dst, int64_t d_t, int64_t d_h,
                                                        int64_t tok0, int n_blk, int hkv,
                                                        int words_per_row, int y0) {
  const int64_t n_words = static_cast<int64_t>(n_blk) * hkv * words_per_row;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n_words) return;
  const bool is_v = blockIdx.y + y0 == 1;
  const int w = static_cast<int>(i % words_per_row);
  const int64_t row = i / words_per_row;
  const int h = static_cast<int>(row % hkv);
  const int64_t t = row / hkv;
  const char* src = is_v ? v_src + t * vs_t + h * vs_h : k_src + t * ks_t + h * ks_h;
  char* dst = (is_v ? v_dst : k_dst) + (tok0 + t) * d_t + h * d_h;
  const u32x4v x = reinterpret_cast<const u32x4v*>(src)[w];
  reinterpret_cast<u32x4v*>(dst)[w] = x;
}

}  // namespace

hipError_t launch_kv_append(const void* k_src, int64_t ks_t, int64_t ks_h, const void* v_src,
                            int64_t vs_t, int64_t vs_h, void* k_dst, void* v_dst, int64_t d_t,
                            int64_t d_h, int64_t tok0, int n_blk, int hkv, int row_bytes,
                            hipStream_t s) {
  const int words = row_bytes / 16;
  const int64_t n_words = static_cast<int64_t>(n_blk) * hkv * words;
  if (n_words == 0) return hipSuccess;
  // grid.y + y0: 0 = K, 1 = V; a NULL source skips that half (its rows are
  // already in place)
  const unsigned y0 = k_src ? 0u : 1u, y1 = v_src ? 2u : 1u;
  if (y1 <= y0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n_words + 255) / 256), y1 - y0);
  hipLaunchKernelGGL(kv_append_kernel, grid, dim3(256), 0, s, static_cast<const char*>(k_src), ks_t,
                     ks_h, static_cast<const char*>(v_src), vs_t, vs_h, static_cast<char*>(k_dst),
                     static_cast<char*>(v_dst), d_t, d_h, tok0, n_blk, hkv, words,
                     static_cast<int>(y0));
  return hipGetLastError();
}

}  // namespace fb
