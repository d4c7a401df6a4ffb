// k1_prefix.hip -- the block-external pass over J_out (the static prefix KV
// cache): A_out and its log-normaliser L_out = ln Z_out for every block query
// row, as cached by FlashBlock (technical summary, s2 "core mechanism").
//
// The prefix is split over the key axis into chunks (split-K); every chunk
// yields a normalised partial (A_c, L_c), and the partials are combined by
// the same log-space composition the method uses for A_full (s2, the A_full
// equation), in a fixed chunk order, so results are run-to-run identical.
//
// Kernels:
//  * prefix_mfma_kernel   bf16, d = 128, few query rows per KV head (the
//    decode regime of text block diffusion: rows = B * Hq/Hkv <= 32 per
//    workgroup row-slab). Grouped-query heads share every K/V tile, which is
//    read from HBM once per KV head. Scores and P.V run on gfx950 MFMA.
//  * prefix_pair_kernel   the same for 33..64 rows per slab: wave pairs share
//    each tile through LDS, each wave computing 32 of the rows.
//  * prefix_generic_kernel  any dtype / d in {64,128} / any row count; VALU.
//    Also implements the sparse SPLIT and GATHER modes.
//  * prefix_reduce_kernel / prefix_reduce_lean_kernel   fixed-order merge of
//    the chunk partials (few rows: 256 threads per row; many rows: 128).
#include "fb_internal.h"

#include <math.h>

namespace fb {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// ---------------------------------------------------------------------------
// Page-selection helpers (sparse modes).
// ---------------------------------------------------------------------------
// Is `page` in the ascending list pages[0..k)?
__device__ __forceinline__ bool page_selected(const int32_t* pages, int k, int32_t page) {
  int lo = 0, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int32_t v = pages[mid];
    if (v == page) return true;
    if (v < page) lo = mid + 1; else hi = mid;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Generic VALU prefix kernel: one wave per (chunk, query row). Lane j scores
// token base + j; the 64 weights are broadcast through LDS for the P.V sum.
// Dense and SPLIT chunk the token axis; GATHER chunks the row's list of
// selected pages (k_pages * page_size virtual tokens).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void prefix_generic_kernel(PrefixParams p) {
  constexpr int NPL = D / 64;                 // dims per lane
  if (p.decide_on && text_step_reuse(p.decide, blockIdx.x == 0 && blockIdx.y == 0)) return;
  const int chunk = blockIdx.x;
  const int64_t row = blockIdx.y;             // t * Hq + h
  const int t = static_cast<int>(row / p.hq);
  const int h = static_cast<int>(row % p.hq);
  if (p.mask && p.mask[h]) return;
  const bool gather = p.sel_mode == FB_SEL_GATHER;
  const bool split = p.sel_mode == FB_SEL_SPLIT;
  if (gather && p.active && !p.active[t]) return;
  const int g = h / p.group;
  const int lane = threadIdx.x;

  __shared__ float qs[D];
  __shared__ float ps[64];
  const T* qrow = static_cast<const T*>(p.q) + t * p.q_st + static_cast<int64_t>(h) * p.q_sh;
  for (int c = lane; c < D; c += 64) qs[c] = to_f32<T>(qrow[c]);
  __syncthreads();

  const T* kbase = static_cast<const T*>(p.k) + static_cast<int64_t>(g) * p.kv_sh;
  const T* vbase = static_cast<const T*>(p.v) + static_cast<int64_t>(g) * p.kv_sh;
  const int32_t* rpages = (split || gather)
      ? p.pages + (static_cast<int64_t>(t) * p.hkv + g) * p.k_pages : nullptr;

  const int64_t n_virt = gather ? static_cast<int64_t>(p.k_pages) * p.page_size : p.n_kv;
  const int64_t per = p.tiles_per_chunk * 64;
  const int64_t lo = static_cast<int64_t>(chunk) * per;
  const int64_t hi = lo + per < n_virt ? lo + per : n_virt;

  auto token_of = [&](int64_t j) -> int64_t {   // virtual -> prefix token, -1 if none
    if (!gather) return j;
    const int64_t tok = static_cast<int64_t>(rpages[j / p.page_size]) * p.page_size + j % p.page_size;
    return tok >= 0 && tok < p.n_kv ? tok : -1;
  };

  const int nsets = split ? 2 : 1;
  float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
  float o[2][NPL];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < NPL; ++i) o[s][i] = 0.f;

  for (int64_t base = lo; base < hi; base += 64) {
    const int64_t j = base + lane;
    int64_t tok = j < hi ? token_of(j) : -1;
    float sc = kNegInf;
    int set = 0;
    if (tok >= 0) {
      const T* kr = kbase + tok * p.kv_st;
      float acc = 0.f;
#pragma unroll 8
      for (int c = 0; c < D; ++c) acc += qs[c] * to_f32<T>(kr[c]);
      sc = acc * p.scale_log2;
      if (split) set = page_selected(rpages, p.k_pages, static_cast<int32_t>(tok / p.page_size)) ? 0 : 1;
    }
    for (int s = 0; s < nsets; ++s) {
      const float x = (set == s) ? sc : kNegInf;
      const float mx = wave_max(x);
      const float mnew = fmaxf(m[s], mx);
      if (mnew == kNegInf) continue;             // wave-uniform
      const float alpha = fast_exp2(m[s] - mnew);
      const float pr = fast_exp2(x - mnew);
      l[s] = l[s] * alpha + wave_sum(pr);
#pragma unroll
      for (int i = 0; i < NPL; ++i) o[s][i] *= alpha;
      m[s] = mnew;
      ps[lane] = pr;
      __syncthreads();
      const int nb = static_cast<int>(hi - base < 64 ? hi - base : 64);
      for (int jj = 0; jj < nb; ++jj) {
        const float pj = ps[jj];
        if (pj == 0.f) continue;                 // wave-uniform
        const int64_t tj = token_of(base + jj);
        const T* vr = vbase + tj * p.kv_st;
#pragma unroll
        for (int i = 0; i < NPL; ++i) o[s][i] += pj * to_f32<T>(vr[lane + 64 * i]);
      }
      __syncthreads();
    }
  }

  for (int s = 0; s < nsets; ++s) {
    const RowOut& out = s == 0 ? p.out : p.out_res;
    const int64_t orow = static_cast<int64_t>(chunk) * out.chunk_stride_rows + row;
    const bool any = l[s] > 0.f;
    const float inv = any ? 1.f / l[s] : 0.f;
#pragma unroll
    for (int i = 0; i < NPL; ++i) out.a[orow * D + lane + 64 * i] = o[s][i] * inv;
    if (lane == 0) out.l[orow] = any ? (m[s] + __log2f(l[s])) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// MFMA prefix kernel (bf16, d = 128).
//
// Workgroup = 4 waves = (chunk of the prefix, KV head g, row slab of 64 rows).
// Rows are the (query token, query head) pairs of the group: r = t*G + j, so
// every K/V byte of the group is read from HBM once for all its query heads.
// Each wave streams its own 32-token tiles of the chunk (tiles w, w+4, ...),
// keeps its own online-softmax state, and the four states are merged through
// LDS at the end. Per tile:
//   global -> VGPR: coalesced 16 B per lane (4 token rows x 256 B per load),
//       non-temporal, addressed as a wave-uniform SGPR base + one VGPR lane
//       offset; DEPTH tiles are in flight per wave (DEPTH x 16 KB of VGPRs);
//   VGPR -> wave-private LDS with padded rows (K: 272 B, V: 320 B), chosen so
//       the operand reads below hit distinct LDS banks;
//   S^T[32 tok x 32 rows] = K . Q^T  (v_mfma_f32_32x32x16_bf16, 8 k-steps)
//       -> each lane owns one row and 16 of its scores: the row max needs
//          one exchange with the other lane half, the row sum none;
//   O^T[128 dims x 32 rows] += V^T . P^T: P^T is the score accumulator itself
//       (as bf16 hi + lo), V^T comes from LDS by ds_read_b64_tr_b16.
// The running row max is raised only when a tile's max exceeds it by more
// than 2^8 (weights then stay <= 256), so most tiles skip the O rescale.
// ---------------------------------------------------------------------------
#ifndef FB_PREFIX_DEPTH_R1
#define FB_PREFIX_DEPTH_R1 1      // tiles in flight per wave, 32-row slabs
#endif
#ifndef FB_PREFIX_DEPTH_R2
#define FB_PREFIX_DEPTH_R2 1      // tiles in flight per wave, 64-row slabs
#endif
#ifndef FB_PREFIX_OCC_R1
#define FB_PREFIX_OCC_R1 1        // workgroups per CU the 32-row kernel is built for
#endif
constexpr int kWaves = 4;
constexpr int kTile = 32;
constexpr int kD = 128;
constexpr int kKRow = 272;                   // 17 x 16 B: 16 rows, 16 bank groups
constexpr int kVRow = 320;                   // 20 x 16 B: 4 rows, 4 x 64 B bank spans
constexpr int kKBytes = kTile * kKRow;
constexpr int kVBytes = kTile * kVRow;
constexpr int kWaveLds = kKBytes + kVBytes;
constexpr float kRescaleLog2 = 8.f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// K/V are streamed once per pass: non-temporal loads (measured on MI355X:
// ~10-15% more read bandwidth than plain loads for this access pattern).
__device__ __forceinline__ u32x4 ldnt(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

struct KvTile {            // one 32-token K/V tile, 16 B per lane per row-load
  u32x4 k[8], v[8];        // native vectors (plain loads, kept in VGPRs)
};

// Transposing LDS read (gfx950): within each 16-lane group, "row" s is the
// concatenation of the 4-element loads of lanes 4s..4s+3, and lane j receives
// element j of rows 0..3. The argument points into __shared__ memory.
__device__ __forceinline__ bf16x4 ds_read_tr(const char* lds_generic) {
  auto p = (const __attribute__((address_space(3))) char*)(lds_generic);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// One 32-token tile for NRB 32-row blocks: S^T = K . Q^T on MFMA, the online
// softmax per row (lane pair l, l^32), O^T += V^T . P^T with the weights as
// bf16 hi + lo parts (two MFMAs: ~2^-16 relative instead of bf16's 2^-8; the
// row sum l is accumulated from the fp32 weights). `valid` = tokens of the
// tile that exist (scores of the others are masked). k_rd / v_rd are this
// lane's LDS operand addresses (see the kernels for the layout).
template <int NRB>
__device__ __forceinline__ void tile_compute(f32x16 (&o)[NRB][4], float (&m_run)[NRB],
                                             float (&l_run)[NRB], const bf16x8 (&qop)[NRB][8],
                                             const char* k_rd, const char* v_rd, float scale_log2,
                                             int64_t valid, int hl) {
  // S^T = K . Q^T
  f32x16 s[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) s[rb] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(k_rd + 32 * kk);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) s[rb] = mfma32(ka, qop[rb][kk], s[rb]);
  }

  // online softmax per row (= lane pair l, l^32); weights enter P.V as
  // bf16 hi + lo parts (two MFMAs: ~2^-16 relative instead of bf16's
  // 2^-8), the row sum l is accumulated from the fp32 weights.
  bf16x8 pbh[NRB][2], pbl[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    // raw scores: the scale c > 0 enters once per score as an fma in the
    // exponent, and max(c s) = c max(s)
    float x[16];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = s[rb][i];
    if (valid < kTile) {               // ragged last tile only
      int vv = static_cast<int>(valid);
      asm volatile("" : "+v"(vv));     // keeps the per-key compares inside the branch
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tk = 8 * (i >> 2) + 4 * hl + (i & 3);
        if (tk >= vv) x[i] = kNegInf;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * scale_log2;
    const bool bump = mx > m_run[rb] + kRescaleLog2;
    float alpha = 1.f;
    if (bump) {
      alpha = fast_exp2(m_run[rb] - mx);
      m_run[rb] = mx;
    }
    const float muse = m_run[rb] == kNegInf ? 0.f : m_run[rb];
    float psum = 0.f;
#pragma unroll
    for (int hj = 0; hj < 2; ++hj) {
      f32x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pf[e] = fast_exp2(fmaf(x[8 * hj + e], scale_log2, -muse));
        psum += pf[e];
      }
      const bf16x8 hi = __builtin_convertvector(pf, bf16x8);
      pbh[rb][hj] = hi;
      pbl[rb][hj] = bf16_lo_part(pf, hi);
    }
    l_run[rb] = l_run[rb] * alpha + psum;
    if (__any(bump)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[rb][db] *= alpha;
    }
  }

  // O^T += V^T . P^T
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bf16x4 v0 = ds_read_tr(v_rd + (16 * j) * kVRow + 64 * db);
      const bf16x4 v1 = ds_read_tr(v_rd + (16 * j + 8) * kVRow + 64 * db);
      // whole-vector concatenation (element-wise inserts of the
      // transposed halves were mis-lowered by the compiler)
      const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        o[rb][db] = mfma32(va, pbh[rb][j], o[rb][db]);
        o[rb][db] = mfma32(va, pbl[rb][j], o[rb][db]);
      }
    }
  }

  asm volatile("" ::: "memory");
}

template <int NRB, int DEPTH, int OCC>
__global__ __launch_bounds__(256, OCC) void prefix_mfma_kernel(PrefixParams p) {
  constexpr int RP = 32 * NRB;                     // padded rows per slab
  constexpr int kStageBytes = kWaves * kWaveLds;
  constexpr int kMergeStride = kD + 1;             // floats per merge row
  constexpr int kMergeBytes = kWaves * RP * kMergeStride * 4;
  constexpr int kLdsBytes = kMergeBytes > kStageBytes ? kMergeBytes : kStageBytes;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  __shared__ float ml_s[kWaves][RP][2];

  if (p.decide_on && text_step_reuse(p.decide, blockIdx.x == 0 && threadIdx.x < 64)) return;
  // XCD-aware order: consecutive workgroup ids go to different XCDs (id mod 8),
  // so the row slabs of one (chunk, KV head) get ids congruent mod 8 and run
  // side by side on one XCD, where the second slab's K/V reads hit its L2.
  int chunk, g, slab;
  {
    const int id = blockIdx.x;
    const int tq = id >> 3;
    slab = tq % p.n_slabs;
    const int idx = (tq / p.n_slabs) * 8 + (id & 7);
    if (idx >= p.n_chunks * p.hkv) return;
    chunk = p.heads_inner ? idx / p.hkv : idx % p.n_chunks;
    g = p.heads_inner ? idx % p.hkv : idx / p.n_chunks;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, r32 = lane & 31;
  const int G = p.group;
  const int R = p.n_q * G;
  const int row0 = slab * RP;

  if (p.mask) {                                    // whole group reused?
    bool all = true;
    for (int j = 0; j < G; ++j) all = all && p.mask[g * G + j] != 0;
    if (all) return;
  }

  // Q^T operands: lane holds row (row0 + 32 rb + r32), dims 16 kk + 8 hl .. +8.
  bf16x8 qop[NRB][8];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = row0 + 32 * rb + r32;
    const bool ok = r < R;
    const int t = ok ? r / G : 0, jh = ok ? r % G : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + static_cast<int64_t>(t) * p.q_st +
                         static_cast<int64_t>(g * G + jh) * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qop[rb][kk] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * hl) : bf16x8{};
  }

  const int64_t n_tiles = (p.n_kv + kTile - 1) / kTile;
  const int64_t t_begin = static_cast<int64_t>(chunk) * p.tiles_per_chunk;
  const int64_t t_end = t_begin + p.tiles_per_chunk < n_tiles ? t_begin + p.tiles_per_chunk : n_tiles;
  if (t_begin >= t_end) return;                    // (every launched chunk has a tile)

  // LDS addresses: one base per access kind, everything else immediates.
  char* kl = lds + w * kWaveLds;
  char* vl = kl + kKBytes;
  const int lrow = lane >> 4, lpiece = lane & 15;
  char* k_wr = kl + lrow * kKRow + lpiece * 16;
  char* v_wr = vl + lrow * kVRow + lpiece * 16;
  const char* k_rd = kl + r32 * kKRow + hl * 16;
  const int grp = lane >> 4, s4 = (lane & 15) >> 2, q4 = lane & 3;
  const char* v_rd = vl + (4 * (grp >> 1) + s4) * kVRow + 32 * (grp & 1) + 8 * q4;

  // global addressing: wave-uniform tile base + one 32-bit lane offset
  const char* kg = static_cast<const char*>(p.k) + static_cast<int64_t>(g) * p.kv_sh * 2;
  const char* vg = static_cast<const char*>(p.v) + static_cast<int64_t>(g) * p.kv_sh * 2;
  const int64_t kvst_b = p.kv_st * 2;
  const uint32_t voff = static_cast<uint32_t>(lrow * kvst_b) + lpiece * 16;

  f32x16 o[NRB][4];
  float m_run[NRB], l_run[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[rb][db] = f32x16{};
  }

  // Every stage is refilled unconditionally (the tile index is clamped to the
  // chunk's last tile once past the end, a re-read that hits L2; rows past
  // n_kv are clamped to the last token, and their scores are masked), so each
  // path through the loop issues the same loads and the waits before staging
  // only cover the stage being consumed.
  const int64_t t_last = t_end - 1;
  auto load_tile = [&](int64_t tile) -> KvTile {
    KvTile r;
    tile = tile < t_last ? tile : t_last;
    const int64_t tok0 = tile * kTile;
    const char* kb = kg + tok0 * kvst_b;
    const char* vb = vg + tok0 * kvst_b;
    if (tok0 + kTile <= p.n_kv) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        r.k[i] = ldnt(kb + 4 * i * kvst_b + voff);
        r.v[i] = ldnt(vb + 4 * i * kvst_b + voff);
      }
    } else {
      const int64_t last = p.n_kv - 1 - tok0;        // >= 0
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t rr = 4 * i + lrow < last ? 4 * i + lrow : last;
        const int64_t off = rr * kvst_b + lpiece * 16;
        r.k[i] = ldnt(kb + off);
        r.v[i] = ldnt(vb + off);
      }
    }
    return r;
  };
  KvTile stage[DEPTH];

  const int64_t tile0 = t_begin + w;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) stage[d] = load_tile(tile0 + d * kWaves);

  auto stage_to_lds = [&](const KvTile& st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(k_wr + 4 * i * kKRow) = st.k[i];
      *reinterpret_cast<u32x4*>(v_wr + 4 * i * kVRow) = st.v[i];
    }
    asm volatile("" ::: "memory");
  };

  auto process = [&](int64_t tile) {
    tile_compute<NRB>(o, m_run, l_run, qop, k_rd, v_rd, p.scale_log2, p.n_kv - tile * kTile, hl);
  };

  // Steady state: whole iterations only, so every stage is consumed and
  // refilled on every path and the wait before staging covers one stage.
  int64_t base = tile0;
  for (; base + (DEPTH - 1) * kWaves < t_end; base += DEPTH * kWaves) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int64_t tile = base + d * kWaves;
      stage_to_lds(stage[d]);
      stage[d] = load_tile(tile + DEPTH * kWaves);
      process(tile);
    }
  }
  // Drain: the last (< DEPTH) tiles of this wave are already staged.
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    const int64_t tile = base + d * kWaves;
    if (tile < t_end) {
      stage_to_lds(stage[d]);
      process(tile);
    }
  }

  // ---- merge the four waves' states through LDS, write the chunk partial --
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) l_run[rb] += __shfl_xor(l_run[rb], 32, 64);
  __syncthreads();                                  // staging LDS no longer read
  if (hl == 0) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      ml_s[w][32 * rb + r32][0] = m_run[rb];
      ml_s[w][32 * rb + r32][1] = l_run[rb];
    }
  }
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = 32 * rb + r32;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, ml_s[ww][r][0]);
    float tot = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = ml_s[ww][r][0];
      if (mw != kNegInf) tot += ml_s[ww][r][1] * fast_exp2(mw - M);
    }
    const float f = (m_run[rb] == kNegInf || tot == 0.f) ? 0.f : fast_exp2(m_run[rb] - M) / tot;
    float* dst = mg + (w * RP + r) * kMergeStride;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[32 * db + 8 * (i >> 2) + 4 * hl + (i & 3)] = o[rb][db][i] * f;
  }
  __syncthreads();

  const int rows_here = R - row0 < RP ? R - row0 : RP;
  for (int e = tid; e < rows_here * kD; e += 256) {
    const int r = e / kD, c = e % kD;
    const int rr = row0 + r;
    const int t = rr / G, jh = rr % G, h = g * G + jh;
    if (p.mask && p.mask[h]) continue;
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) sum += mg[(ww * RP + r) * kMergeStride + c];
    const int64_t orow = static_cast<int64_t>(chunk) * p.out.chunk_stride_rows +
                         static_cast<int64_t>(t) * p.hq + h;
    p.out.a[orow * kD + c] = sum;
  }
  for (int r = tid; r < rows_here; r += 256) {
    const int rr = row0 + r;
    const int t = rr / G, jh = rr % G, h = g * G + jh;
    if (p.mask && p.mask[h]) continue;
    float M = kNegInf;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, ml_s[ww][r][0]);
    float tot = 0.f;
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = ml_s[ww][r][0];
      if (mw != kNegInf) tot += ml_s[ww][r][1] * fast_exp2(mw - M);
    }
    const int64_t orow = static_cast<int64_t>(chunk) * p.out.chunk_stride_rows +
                         static_cast<int64_t>(t) * p.hq + h;
    p.out.l[orow] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Row-split MFMA prefix kernel: 33..64 query rows per KV head (a 16-token block
// of a 4:1 grouped-query model has 64). An 8-wave workgroup forms NP = 4
// pairs; each pair streams every fourth tile of the chunk into its own
// double-buffered LDS region -- one wave of the pair stages the tile's K, the
// other its V -- and each wave of the pair computes 32 of the 64 rows from
// the shared tile. One barrier per tile orders the stores of tile k against
// the reads of tile k-1 of the other buffer. Per-wave state is that of 32
// rows; one workgroup (8 waves, 151 KB of LDS) per CU, and every K/V byte
// still crosses HBM once. Four streams per workgroup instead of two halve
// the split-K partials (measured at 131k tokens: 102.9 -> 93.7 us).
// ---------------------------------------------------------------------------
#ifndef FB_PREFIX_DEPTH_PAIR
#define FB_PREFIX_DEPTH_PAIR 1    // half-tiles in flight per wave
#endif
#ifndef FB_PREFIX_NP
#define FB_PREFIX_NP 4            // wave pairs (tile streams) per workgroup
#endif
#ifndef FB_PREFIX_OCC_PAIR
#define FB_PREFIX_OCC_PAIR 1      // workgroups per CU
#endif
constexpr int kPairBuf = kKBytes + kVBytes;       // one K+V tile in LDS
constexpr int kBufDword3 = 0x00020000;            // buffer resource word 3 (gfx9 raw buffer)
constexpr int kAuxNT = 2;                         // cache policy: non-temporal

struct HalfTile {          // the K (or V) half of a tile: 8 row-loads per lane
  u32x4 r[8];
};

template <int DEPTH, int OCC, int NP>
__global__ __launch_bounds__(128 * NP, OCC) void prefix_pair_kernel(PrefixParams p) {
  constexpr int NT = 128 * NP;                     // threads: NP pairs of waves
  constexpr int kStageBytes = NP * 2 * kPairBuf;   // NP pairs x 2 buffers
  constexpr int kMergeStride = kD + 1;
  constexpr int kMergeBytes = 2 * NP * 32 * kMergeStride * 4;
  constexpr int kLdsBytes = kMergeBytes > kStageBytes ? kMergeBytes : kStageBytes;
  constexpr int U = 2 * DEPTH;                     // unroll: static stage and buffer index
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  __shared__ float ml_s[2 * NP][32][2];

  if (p.decide_on && text_step_reuse(p.decide, blockIdx.x == 0 && threadIdx.x < 64)) return;
  int chunk, g, slab;
  {
    const int id = blockIdx.x;
    const int tq = id >> 3;
    slab = tq % p.n_slabs;
    const int idx = (tq / p.n_slabs) * 8 + (id & 7);
    if (idx >= p.n_chunks * p.hkv) return;
    chunk = p.heads_inner ? idx / p.hkv : idx % p.n_chunks;
    g = p.heads_inner ? idx % p.hkv : idx / p.n_chunks;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w >> 1, hr = w & 1;             // tile stream, row block / K-or-V role
  const int hl = lane >> 5, r32 = lane & 31;
  const int G = p.group;
  const int R = p.n_q * G;
  const int row0 = slab * 64;
  const bool rows_live = row0 + 32 * hr < R;       // this wave's row block has rows

  if (p.mask) {
    bool all = true;
    for (int j = 0; j < G; ++j) all = all && p.mask[g * G + j] != 0;
    if (all) return;
  }

  bf16x8 qop[1][8];
  {
    const int r = row0 + 32 * hr + r32;
    const bool ok = r < R;
    const int t = ok ? r / G : 0, jh = ok ? r % G : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + static_cast<int64_t>(t) * p.q_st +
                         static_cast<int64_t>(g * G + jh) * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qop[0][kk] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * hl) : bf16x8{};
  }

  const int64_t n_tiles = (p.n_kv + kTile - 1) / kTile;
  // Groups of NP tiles are dealt round-robin over the chunks (iteration it
  // of pair q is tile NP (chunk + n_chunks it) + q): the workgroups of a KV
  // head walk the prefix side by side, one sequential stream per head and
  // K/V instead of one per chunk (measured 1-4% faster on a head-major cache
  // than contiguous chunks). The plan keeps NP n_chunks <= n_tiles, so every
  // chunk has a tile.
  const int64_t t_begin = NP * static_cast<int64_t>(chunk);
  const int64_t t_step = NP * static_cast<int64_t>(p.n_chunks);
  const int64_t t_end = n_tiles;
  if (t_begin >= t_end) return;
  const int64_t n_iter = (t_end - t_begin + t_step - 1) / t_step;

  // LDS: pair region = 2 buffers x (K tile, V tile)
  char* pbase = lds + pair * 2 * kPairBuf;
  const int lrow = lane >> 4, lpiece = lane & 15;
  const int grp = lane >> 4, s4 = (lane & 15) >> 2, q4 = lane & 3;
  char* wr = pbase + (hr == 0 ? lrow * kKRow : kKBytes + lrow * kVRow) + lpiece * 16;
  const char* k_rd = pbase + r32 * kKRow + hl * 16;
  const char* v_rd = pbase + kKBytes + (4 * (grp >> 1) + s4) * kVRow + 32 * (grp & 1) + 8 * q4;

  // Global reads through a buffer resource rebuilt per tile (scalar work):
  // its record count ends at the last token of the prefix, so the rows of a
  // ragged last tile past n_kv read as zeros, and a prefetch past the chunk's
  // last tile (record count 0) reads nothing at all. Each lane keeps one
  // 32-bit offset per row-load.
  const char* src = static_cast<const char*>(hr == 0 ? p.k : p.v) +
                    static_cast<int64_t>(g) * p.kv_sh * 2;
  const int64_t kvst_b = p.kv_st * 2;
  uint32_t voffs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    voffs[i] = static_cast<uint32_t>((4 * i + lrow) * kvst_b) + lpiece * 16;

  auto load_half = [&](int64_t it) -> HalfTile {   // this wave's half of pair tile `it`
    HalfTile r;
    const int64_t tile = t_begin + t_step * it + pair;
    const int64_t tok0 = tile * kTile;
    const int64_t rows = tile < t_end ? (p.n_kv - tok0 < kTile ? p.n_kv - tok0 : kTile) : 0;
    const int nrec = rows > 0 ? static_cast<int>((rows - 1) * kvst_b) + kD * 2 : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(src + (tile < t_end ? tok0 : 0) * kvst_b), 0, nrec, kBufDword3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      r.r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voffs[i]), 0, kAuxNT);
    return r;
  };

  // LDS row stride as an immediate: one store sequence per role (wave-uniform)
  auto store_half = [&](const HalfTile& h, int boff) {
    if (hr == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(wr + boff + 4 * i * kKRow) = h.r[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(wr + boff + 4 * i * kVRow) = h.r[i];
    }
  };

  f32x16 o[1][4];
  float m_run[1] = {kNegInf}, l_run[1] = {0.f};
#pragma unroll
  for (int db = 0; db < 4; ++db) o[0][db] = f32x16{};

  HalfTile stage[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) stage[d] = load_half(d);

  auto iteration = [&](int u, int64_t it) {      // u static: stage u % DEPTH, buffer u % 2
    const int boff = (u & 1) * kPairBuf;
    store_half(stage[u % DEPTH], boff);
    stage[u % DEPTH] = load_half(it + DEPTH);
    __syncthreads();
    const int64_t tile = t_begin + t_step * it + pair;
    if (tile < t_end && rows_live)
      tile_compute<1>(o, m_run, l_run, qop, k_rd + boff, v_rd + boff, p.scale_log2,
                      p.n_kv - tile * kTile, hl);
  };

  int64_t it = 0;
  for (; it + U <= n_iter; it += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) iteration(u, it + u);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (it + u < n_iter) iteration(u, it + u);      // workgroup-uniform

  // ---- merge the NP tile streams of each row block, write the partial ----
  // (row block hr of stream q lives in wave 2 q + hr)
  l_run[0] += __shfl_xor(l_run[0], 32, 64);
  __syncthreads();
  if (hl == 0) {
    ml_s[w][r32][0] = m_run[0];
    ml_s[w][r32][1] = l_run[0];
  }
  __syncthreads();
  float* mg = reinterpret_cast<float*>(lds);
  {
    float M = kNegInf;
#pragma unroll
    for (int q = 0; q < NP; ++q) M = fmaxf(M, ml_s[2 * q + hr][r32][0]);
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const float mq = ml_s[2 * q + hr][r32][0];
      if (mq != kNegInf) tot += ml_s[2 * q + hr][r32][1] * fast_exp2(mq - M);
    }
    const float f = (m_run[0] == kNegInf || tot == 0.f) ? 0.f : fast_exp2(m_run[0] - M) / tot;
    float* dst = mg + (w * 32 + r32) * kMergeStride;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[32 * db + 8 * (i >> 2) + 4 * hl + (i & 3)] = o[0][db][i] * f;
  }
  __syncthreads();

  const int rows_here = R - row0 < 64 ? R - row0 : 64;
  for (int e = tid; e < rows_here * kD; e += NT) {
    const int r = e / kD, c = e % kD;
    const int rr = row0 + r;
    const int t = rr / G, jh = rr % G, h = g * G + jh;
    if (p.mask && p.mask[h]) continue;
    const int rb = r >> 5, rl = r & 31;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) sum += mg[((2 * q + rb) * 32 + rl) * kMergeStride + c];
    const int64_t orow = static_cast<int64_t>(chunk) * p.out.chunk_stride_rows +
                         static_cast<int64_t>(t) * p.hq + h;
    p.out.a[orow * kD + c] = sum;
  }
  for (int r = tid; r < rows_here; r += NT) {
    const int rr = row0 + r;
    const int t = rr / G, jh = rr % G, h = g * G + jh;
    if (p.mask && p.mask[h]) continue;
    const int rb = r >> 5, rl = r & 31;
    float M = kNegInf;
#pragma unroll
    for (int q = 0; q < NP; ++q) M = fmaxf(M, ml_s[2 * q + rb][rl][0]);
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const float mq = ml_s[2 * q + rb][rl][0];
      if (mq != kNegInf) tot += ml_s[2 * q + rb][rl][1] * fast_exp2(mq - M);
    }
    const int64_t orow = static_cast<int64_t>(chunk) * p.out.chunk_stride_rows +
                         static_cast<int64_t>(t) * p.hq + h;
    p.out.l[orow] = tot > 0.f ? (M + __log2f(tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Split-K reduce: merge the chunk partials of every (query, head) row with the
// A_full composition rule (weights e^{L_c - max L}). One workgroup per row:
// the chunk weights are computed once into LDS, then every dim sums its
// chunks with independent (unrolled) loads; all sums run in a fixed order.
// SPLIT: a_out merges selected + residual partials, a_res the residual ones.
// GATHER: a_out merges the selected partials with the cached residual input.
// ---------------------------------------------------------------------------
constexpr int kMaxChunks = 1024;
constexpr int64_t kReduceLeanRows = 4096;    // rows from which the lean reduce runs


// One workgroup (256 threads) per output row. Thread (half, c) sums dim c
// over its half of the chunks with every load of the half in flight at
// once, and the two halves meet in LDS; the chunk weights come from one
// wave's max. The chunk order of every sum is fixed, so results are
// run-to-run identical.
// The row's query copy (ReduceParams.q_src), one 32-bit word per thread.
__device__ __forceinline__ void copy_row_query(const ReduceParams& p, int t, int h) {
  if (!p.q_src) return;
  const int words = p.d * p.q_esize / 4;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(
      static_cast<const char*>(p.q_src) + (t * p.q_st + h * p.q_sh) * p.q_esize);
  uint32_t* dst = reinterpret_cast<uint32_t*>(
      static_cast<char*>(p.q_dst) + (static_cast<int64_t>(t) * p.hq + h) * p.d * p.q_esize);
  for (int i = threadIdx.x; i < words; i += blockDim.x) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void prefix_reduce_kernel(ReduceParams p) {
  __shared__ float wa[kMaxChunks];
  __shared__ float wr[kMaxChunks + 1];
  __shared__ float red[4];
  __shared__ float half_acc[2][2][128];            // [half][set][dim]
  const int64_t row = blockIdx.x;
  const int h = static_cast<int>(row % p.hq);
  const int t = static_cast<int>(row / p.hq);
  copy_row_query(p, t, h);
  if (p.mask && p.mask[h]) return;
  if (p.active && !p.active[t]) return;
  const int tid = threadIdx.x;
  const int nc = p.dyn.on ? rows_dyn_split(groups_on(p.mask, p.dyn.hkv, p.dyn.group), p.dyn).chunks
                          : p.n_chunks;
  const int nr = p.part_rl ? nc : 0;               // residual partials (SPLIT)
  const bool cached = p.res_l != nullptr;          // cached residual (GATHER)

  float m = kNegInf, mr = kNegInf;
  for (int ch = tid; ch < nc; ch += 256) m = fmaxf(m, p.part_l[ch * p.rows + row]);
  for (int ch = tid; ch < nr; ch += 256) mr = fmaxf(mr, p.part_rl[ch * p.rows + row]);
  if (cached && tid == 0) mr = fmaxf(mr, p.res_l[row]);
  m = wave_max(m);
  mr = wave_max(mr);
  if ((tid & 63) == 0) {
    red[tid >> 6] = m;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = mr;
  __syncthreads();
  const float Mr = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float Mall = fmaxf(M, Mr);

  for (int ch = tid; ch < nc; ch += 256) {
    const float L = p.part_l[ch * p.rows + row];
    wa[ch] = L == kNegInf ? 0.f : expf(L - Mall);
  }
  for (int ch = tid; ch < nr; ch += 256) {
    const float L = p.part_rl[ch * p.rows + row];
    wr[ch] = L == kNegInf ? 0.f : expf(L - Mr);
  }
  if (cached && tid == 0) {
    const float L = p.res_l[row];
    wr[nr] = L == kNegInf ? 0.f : expf(L - Mr);
  }
  __syncthreads();
  const int nrt = nr + (cached ? 1 : 0);
  float S = 0.f, Sr = 0.f;                         // same order in every thread
  for (int ch = 0; ch < nc; ++ch) S += wa[ch];
  for (int ch = 0; ch < nrt; ++ch) Sr += wr[ch];

  const int hf = tid >> 7, c = tid & 127;          // half of the chunks, dim
  const int64_t cs = p.rows * p.d;                 // chunk stride
  const int mid = (nc + 1) / 2, midr = (nr + 1) / 2;
  if (c < p.d) {
    const int c0 = hf ? mid : 0, c1 = hf ? nc : mid;
    float acc = 0.f;
    const float* pa = p.part_a + row * p.d + c;
    int ch = c0;
    for (; ch + 16 <= c1; ch += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = pa[(ch + u) * cs];
#pragma unroll
      for (int u = 0; u < 16; ++u) acc += wa[ch + u] * v[u];
    }
    for (; ch < c1; ++ch) acc += wa[ch] * pa[ch * cs];
    half_acc[hf][0][c] = acc;
    float accr = 0.f;
    if (nr) {
      const int r0 = hf ? midr : 0, r1 = hf ? nr : midr;
      const float* pr = p.part_ra + row * p.d + c;
      for (ch = r0; ch < r1; ++ch) accr += wr[ch] * pr[ch * cs];
    }
    half_acc[hf][1][c] = accr;
  }
  __syncthreads();
  if (tid < p.d) {
    const float acc = half_acc[0][0][c] + half_acc[1][0][c];
    float accr = half_acc[0][1][c] + half_acc[1][1][c];
    if (cached) accr += wr[nr] * p.res_a[row * p.d + c];
    if (p.a_res) p.a_res[row * p.d + c] = Mr != kNegInf ? accr / Sr : 0.f;
    // fold the residual pair into the full pair (same composition)
    const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
    const float Stot = S + Sr * wrr;
    p.a_out[row * p.d + c] = Mall != kNegInf ? (acc + accr * wrr) / Stot : 0.f;
  }
  if (tid == 0) {
    if (p.a_res) p.l_res[row] = Mr != kNegInf ? Mr + logf(Sr) : kNegInf;
    const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
    p.l_out[row] = Mall != kNegInf ? Mall + logf(S + Sr * wrr) : kNegInf;
  }
}

__device__ __forceinline__ float block_max128(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(red[0], red[1]);
  __syncthreads();
  return r;
}

// Many-row variant (one 128-thread workgroup per row, thread c sums dim c
// over all chunks, 8 loads in flight): with tens of thousands of rows the
// occupancy of the lean workgroup matters more than one row's latency.
__global__ __launch_bounds__(128) void prefix_reduce_lean_kernel(ReduceParams p) {
  __shared__ float wa[kMaxChunks];
  __shared__ float wr[kMaxChunks + 1];
  __shared__ float red[2];
  const int64_t row = blockIdx.x;
  const int h = static_cast<int>(row % p.hq);
  const int t = static_cast<int>(row / p.hq);
  copy_row_query(p, t, h);
  if (p.mask && p.mask[h]) return;
  if (p.active && !p.active[t]) return;
  const int tid = threadIdx.x;
  const int nc = p.dyn.on ? rows_dyn_split(groups_on(p.mask, p.dyn.hkv, p.dyn.group), p.dyn).chunks
                          : p.n_chunks;
  const int nr = p.part_rl ? nc : 0;               // residual partials (SPLIT)
  const bool cached = p.res_l != nullptr;          // cached residual (GATHER)

  float m = kNegInf, mr = kNegInf;
  for (int ch = tid; ch < nc; ch += 128) m = fmaxf(m, p.part_l[ch * p.rows + row]);
  for (int ch = tid; ch < nr; ch += 128) mr = fmaxf(mr, p.part_rl[ch * p.rows + row]);
  if (cached && tid == 0) mr = fmaxf(mr, p.res_l[row]);
  const float M = block_max128(m, red);
  const float Mr = block_max128(mr, red);
  const float Mall = fmaxf(M, Mr);

  for (int ch = tid; ch < nc; ch += 128) {
    const float L = p.part_l[ch * p.rows + row];
    wa[ch] = L == kNegInf ? 0.f : expf(L - Mall);
  }
  for (int ch = tid; ch < nr; ch += 128) {
    const float L = p.part_rl[ch * p.rows + row];
    wr[ch] = L == kNegInf ? 0.f : expf(L - Mr);
  }
  if (cached && tid == 0) {
    const float L = p.res_l[row];
    wr[nr] = L == kNegInf ? 0.f : expf(L - Mr);
  }
  __syncthreads();
  const int nrt = nr + (cached ? 1 : 0);
  float S = 0.f, Sr = 0.f;                         // same order in every thread
  for (int ch = 0; ch < nc; ++ch) S += wa[ch];
  for (int ch = 0; ch < nrt; ++ch) Sr += wr[ch];

  const int c = tid;
  if (c < p.d) {
    float acc = 0.f, accr = 0.f;
    const float* pa = p.part_a + row * p.d + c;
    const int64_t cs = p.rows * p.d;               // chunk stride
    int ch = 0;
    for (; ch + 8 <= nc; ch += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pa[(ch + u) * cs];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += wa[ch + u] * v[u];
    }
    for (; ch < nc; ++ch) acc += wa[ch] * pa[ch * cs];
    if (nr) {
      const float* pr = p.part_ra + row * p.d + c;
      for (ch = 0; ch < nr; ++ch) accr += wr[ch] * pr[ch * cs];
    }
    if (cached) accr += wr[nr] * p.res_a[row * p.d + c];
    if (p.a_res) p.a_res[row * p.d + c] = Mr != kNegInf ? accr / Sr : 0.f;
    // fold the residual pair into the full pair (same composition)
    const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
    const float Stot = S + Sr * wrr;
    p.a_out[row * p.d + c] = Mall != kNegInf ? (acc + accr * wrr) / Stot : 0.f;
  }
  if (tid == 0) {
    if (p.a_res) p.l_res[row] = Mr != kNegInf ? Mr + logf(Sr) : kNegInf;
    const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
    p.l_out[row] = Mall != kNegInf ? Mall + logf(S + Sr * wrr) : kNegInf;
  }
}

// Many-row variant with up to 64 chunks: one wave per row (lane c holds
// chunk c's log-normaliser and weight, lane l dims l, l + 64), 4 waves a
// workgroup, kWaveRows rows a wave. The weights are read back lane by lane in
// chunk order, so every sum has the operations and the order of the
// 128-thread form (the same bits) without its barriers; a workgroup per row
// made the 56,160-row video reduce a dispatch-bound launch.
constexpr int kWaveRows = 2;
constexpr int kWaveMaxChunks = 64;
constexpr int kWavePreChunks = 8;                // chunks whose partials are loaded up front

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__global__ __launch_bounds__(256) void prefix_reduce_wave_kernel(ReduceParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kWaveRows;
  const int nc = p.dyn.on ? rows_dyn_split(groups_on(p.mask, p.dyn.hkv, p.dyn.group), p.dyn).chunks
                          : p.n_chunks;
  const int nr = p.part_rl ? nc : 0;               // residual partials (SPLIT)
  const bool cached = p.res_l != nullptr;          // cached residual (GATHER)
  const int64_t cs = p.rows * p.d;                 // chunk stride
  if (nc <= kWavePreChunks && nr == 0 && p.d <= 128 && !p.q_src) {
    // the usual masked pass (a few chunks): every load of the wave's rows is
    // issued first (nothing for rows past the end or rows the mask or the
    // active flags leave), then each row is formed as below
    float Lv[kWaveRows], Lcv[kWaveRows], rav[kWaveRows][2], av[kWaveRows][kWavePreChunks][2];
    bool on[kWaveRows];
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
      const int64_t row = row0 + r;
      on[r] = row < p.rows && !(p.mask && p.mask[row % p.hq]) &&
              !(p.active && !p.active[row / p.hq]);
    }
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
      const int64_t row = row0 + r;
      if (!on[r]) continue;                        // (uniform in the wave)
      Lv[r] = lane < nc ? p.part_l[lane * p.rows + row] : kNegInf;
      Lcv[r] = cached ? p.res_l[row] : kNegInf;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j < p.d ? lane + 64 * j : 0;
        rav[r][j] = cached ? p.res_a[row * p.d + c] : 0.f;
#pragma unroll
        for (int ch = 0; ch < kWavePreChunks; ++ch)
          av[r][ch][j] = ch < nc ? p.part_a[row * p.d + c + ch * cs] : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
      const int64_t row = row0 + r;
      if (!on[r]) continue;                        // (uniform in the wave)
      const float L = Lv[r], Lc = Lcv[r];
      float mr = kNegInf;
      if (cached && lane == 0) mr = fmaxf(mr, Lc);
      const float M = wave_max(L);
      const float Mr = wave_max(mr);
      const float Mall = fmaxf(M, Mr);
      const float wa = lane < nc ? (L == kNegInf ? 0.f : expf(L - Mall)) : 0.f;
      const float wc = cached ? (Lc == kNegInf ? 0.f : expf(Lc - Mr)) : 0.f;
      float S = 0.f, Sr = 0.f;
      for (int ch = 0; ch < nc; ++ch) S += lane_f(wa, ch);
      if (cached) Sr += wc;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = lane + 64 * j;
        if (c >= p.d) continue;
        float acc = 0.f, accr = 0.f;
#pragma unroll
        for (int ch = 0; ch < kWavePreChunks; ++ch)
          if (ch < nc) acc += lane_f(wa, ch) * av[r][ch][j];
        if (cached) accr += wc * rav[r][j];
        if (p.a_res) p.a_res[row * p.d + c] = Mr != kNegInf ? accr / Sr : 0.f;
        const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
        const float Stot = S + Sr * wrr;
        p.a_out[row * p.d + c] = Mall != kNegInf ? (acc + accr * wrr) / Stot : 0.f;
      }
      if (lane == 0) {
        if (p.a_res) p.l_res[row] = Mr != kNegInf ? Mr + logf(Sr) : kNegInf;
        const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
        p.l_out[row] = Mall != kNegInf ? Mall + logf(S + Sr * wrr) : kNegInf;
      }
    }
    return;
  }
  for (int r = 0; r < kWaveRows; ++r) {
    const int64_t row = row0 + r;
    if (row >= p.rows) return;                     // (uniform in the wave)
    const int h = static_cast<int>(row % p.hq);
    const int t = static_cast<int>(row / p.hq);
    if (p.q_src) {                                 // the row's query copy
      const int words = p.d * p.q_esize / 4;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(
          static_cast<const char*>(p.q_src) + (t * p.q_st + h * p.q_sh) * p.q_esize);
      uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<char*>(p.q_dst) + row * p.d * p.q_esize);
      for (int i = lane; i < words; i += 64) dst[i] = src[i];
    }
    if (p.mask && p.mask[h]) continue;
    if (p.active && !p.active[t]) continue;
    const float L = lane < nc ? p.part_l[lane * p.rows + row] : kNegInf;
    const float Lr = lane < nr ? p.part_rl[lane * p.rows + row] : kNegInf;
    const float Lc = cached ? p.res_l[row] : kNegInf;
    float mr = Lr;
    if (cached && lane == 0) mr = fmaxf(mr, Lc);
    const float M = wave_max(L);
    const float Mr = wave_max(mr);
    const float Mall = fmaxf(M, Mr);
    const float wa = lane < nc ? (L == kNegInf ? 0.f : expf(L - Mall)) : 0.f;
    const float wr = lane < nr ? (Lr == kNegInf ? 0.f : expf(Lr - Mr)) : 0.f;
    const float wc = cached ? (Lc == kNegInf ? 0.f : expf(Lc - Mr)) : 0.f;
    float S = 0.f, Sr = 0.f;                       // chunk order, as in every thread there
    for (int ch = 0; ch < nc; ++ch) S += lane_f(wa, ch);
    for (int ch = 0; ch < nr; ++ch) Sr += lane_f(wr, ch);
    if (cached) Sr += wc;
    for (int c = lane; c < p.d; c += 64) {
      float acc = 0.f, accr = 0.f;
      const float* pa = p.part_a + row * p.d + c;
      int ch = 0;
      for (; ch + 8 <= nc; ch += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pa[(ch + u) * cs];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += lane_f(wa, ch + u) * v[u];
      }
      for (; ch < nc; ++ch) acc += lane_f(wa, ch) * pa[ch * cs];
      if (nr) {
        const float* pr = p.part_ra + row * p.d + c;
        for (ch = 0; ch < nr; ++ch) accr += lane_f(wr, ch) * pr[ch * cs];
      }
      if (cached) accr += wc * p.res_a[row * p.d + c];
      if (p.a_res) p.a_res[row * p.d + c] = Mr != kNegInf ? accr / Sr : 0.f;
      // fold the residual pair into the full pair (same composition)
      const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
      const float Stot = S + Sr * wrr;
      p.a_out[row * p.d + c] = Mall != kNegInf ? (acc + accr * wrr) / Stot : 0.f;
    }
    if (lane == 0) {
      if (p.a_res) p.l_res[row] = Mr != kNegInf ? Mr + logf(Sr) : kNegInf;
      const float wrr = Mr != kNegInf ? expf(Mr - Mall) : 0.f;
      p.l_out[row] = Mall != kNegInf ? Mall + logf(S + Sr * wrr) : kNegInf;
    }
  }
}

__global__ __launch_bounds__(128) void prefix_empty_kernel(float* a, float* l, int hq, int d,
                                                           const uint8_t* mask) {
  const int64_t row = blockIdx.x;
  const int h = static_cast<int>(row % hq);
  if (mask && mask[h]) return;
  if (threadIdx.x < d) a[row * d + threadIdx.x] = 0.f;
  if (threadIdx.x == 0) l[row] = kNegInf;
}

}  // namespace

int prefix_tile_tokens(int path) { return path == 1 ? kTile : 64; }

hipError_t launch_prefix_generic(const PrefixParams& p, fb_dtype dt, int d, hipStream_t s) {
  dim3 grid(p.n_chunks, static_cast<unsigned>(static_cast<int64_t>(p.n_q) * p.hq));
  if (dt == FB_BF16) {
    if (d == 128) hipLaunchKernelGGL((prefix_generic_kernel<uint16_t, 128>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((prefix_generic_kernel<uint16_t, 64>), grid, dim3(64), 0, s, p);
  } else {
    if (d == 128) hipLaunchKernelGGL((prefix_generic_kernel<float, 128>), grid, dim3(64), 0, s, p);
    else hipLaunchKernelGGL((prefix_generic_kernel<float, 64>), grid, dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

int prefix_mfma_occupancy(int row_blocks) {
  return row_blocks == 1 ? FB_PREFIX_OCC_R1 : (row_blocks == 3 ? FB_PREFIX_OCC_PAIR : 1);
}

hipError_t launch_prefix_mfma(const PrefixParams& p, int row_blocks, hipStream_t s) {
  const int n_cg = p.n_chunks * p.hkv;
  dim3 grid(static_cast<unsigned>((n_cg + 7) / 8 * 8 * p.n_slabs));
  if (row_blocks == 1)
    hipLaunchKernelGGL((prefix_mfma_kernel<1, FB_PREFIX_DEPTH_R1, FB_PREFIX_OCC_R1>), grid,
                       dim3(256), 0, s, p);
  else if (row_blocks == 3)        // 64-row slabs split over wave pairs
    hipLaunchKernelGGL((prefix_pair_kernel<FB_PREFIX_DEPTH_PAIR, FB_PREFIX_OCC_PAIR, FB_PREFIX_NP>),
                       grid, dim3(128 * FB_PREFIX_NP), 0, s, p);
  else
    hipLaunchKernelGGL((prefix_mfma_kernel<2, FB_PREFIX_DEPTH_R2, 1>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prefix_reduce(const ReduceParams& p, hipStream_t s) {
  if (p.rows >= kReduceLeanRows && p.n_chunks <= kWaveMaxChunks && p.d <= 128)
    hipLaunchKernelGGL(prefix_reduce_wave_kernel,
                       dim3(static_cast<unsigned>((p.rows + 4 * kWaveRows - 1) / (4 * kWaveRows))),
                       dim3(256), 0, s, p);
  else if (p.rows >= kReduceLeanRows)
    hipLaunchKernelGGL(prefix_reduce_lean_kernel, dim3(static_cast<unsigned>(p.rows)), dim3(128), 0,
                       s, p);
  else
    hipLaunchKernelGGL(prefix_reduce_kernel, dim3(static_cast<unsigned>(p.rows)), dim3(256), 0, s,
                       p);
  return hipGetLastError();
}

hipError_t launch_prefix_empty(float* a_out, float* l_out, int n_q, int hq, int d,
                               const uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(prefix_empty_kernel, dim3(n_q * hq), dim3(128), 0, s, a_out, l_out, hq, d, mask);
  return hipGetLastError();
}

}  // namespace fb
