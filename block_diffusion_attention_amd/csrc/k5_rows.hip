// k5_rows.hip -- attention for many query rows per KV head on MFMA (bf16,
// d = 128): the prefill regime of both passes of the step when a block holds
// thousands of queries (video generation), so that every K/V tile is reused
// by many rows and the work is bound by matrix throughput, not by HBM.
//   * the block-external pass over J_out: A_out and L_out = ln Z_out per row,
//     direct or as split-K partials for the fixed-order reduce (FlashBlock
//     technical summary, s2 "core mechanism");
//   * the block-internal pass over J_in with the log-space composition of the
//     cached pair and the fresh one in its epilogue (s2, the A_full equation).
//
// Workgroup = NW waves = (KV head g, key chunk, row tile of 32 NW RB rows),
// RB 32-row blocks per wave (RB = 1 is the fastest measured: 2 blocks per
// wave with 4 waves, O in accumulation registers, ran slower). Rows are
// (query token, query head of the group) pairs r = t*G + j, so grouped heads
// share every K/V tile. The waves share each 32-key K/V tile, staged global
// -> VGPR -> LDS (eight stages, one barrier per two tiles); each wave keeps the online-softmax state of its rows over the whole
// key range of its chunk, and runs a software pipeline over the tiles: the
// softmax of tile t (VALU) is interleaved with S(t+1) = QK(t+1) and
// O += P(t-1).V(t-1) (matrix core). Per tile and wave:
//   S^T[32 keys x 32 rows] = K . Q^T     (v_mfma_f32_32x32x16_bf16, 8 k-steps;
//       each lane owns one row and 16 of its scores)
//   O^T[128 dims x 32 rows] += V^T . P^T (P^T = the weights as bf16 hi + lo
//       parts, V^T from LDS by the transposing read ds_read_b64_tr_b16)
// The row max is taken on raw scores (scale > 0) and folded into one FMA per
// weight; it is raised only when a tile's max exceeds it by more than 2^8.
// The weights take the running max as it stands, so their exponentials do
// not wait for the tile's max; the rare tile that raises the max recomputes
// its weights (same values as computing them after the raise). The tile loop
// runs two tiles per trip so S(t) and S(t+1) alternate between two register
// sets instead of being copied.
#include "fb_internal.h"

#include <math.h>

namespace fb {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kTile = 32;                    // keys per tile
constexpr int kD = 128;
constexpr int kKRow = 272;                   // 17 x 16 B: 16 rows, 16 bank groups
constexpr int kVRow = 320;                   // 20 x 16 B: 4 rows, 4 x 64 B bank spans
constexpr int kKBytes = kTile * kKRow;
constexpr int kVBytes = kTile * kVRow;
constexpr int kStage = kKBytes + kVBytes;
constexpr float kRescaleLog2 = 8.f;

#ifndef FB_ROWS_VALU_PER
#define FB_ROWS_VALU_PER 6        // VALU instructions issued after each MFMA of a tile
#endif
#ifndef FB_ROWS_WAVES
#define FB_ROWS_WAVES 8           // waves (32 query rows each) per workgroup
#endif
#ifndef FB_ROWS_BLOCKS
#define FB_ROWS_BLOCKS 1          // 32-row blocks per wave
#endif
#ifndef FB_ROWS_OCC
#define FB_ROWS_OCC 1             // workgroups per CU the kernel is built for (register budget)
#endif
#ifndef FB_ROWS_PSPLIT
#define FB_ROWS_PSPLIT 1          // weights as bf16 hi + lo in P.V (0: one bf16 part)
#endif


typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <bool B> struct Flag { static constexpr bool value = B; };
template <int I> struct Int { static constexpr int value = I; };

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read (gfx950): within each 16-lane group, "row" s is the
// concatenation of the 4-element loads of lanes 4s..4s+3, and lane j receives
// element j of rows 0..3.
__device__ __forceinline__ bf16x4 ds_read_tr(const char* lds_generic) {
  auto p = (const __attribute__((address_space(3))) char*)(lds_generic);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
}

// S^T[32 keys x 32 rows] = K . Q^T for one tile and each of the wave's RB
// row blocks; k_rd = this lane's K row. Each K operand is read once and
// feeds the RB blocks' MFMAs.
template <int RB>
__device__ __forceinline__ void qk_tile(const char* k_rd, const bf16x8 (&qop)[RB][8],
                                        f32x16 (&s)[RB]) {
#pragma unroll
  for (int b = 0; b < RB; ++b) s[b] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 k = *reinterpret_cast<const bf16x8*>(k_rd + 32 * kk);
#pragma unroll
    for (int b = 0; b < RB; ++b) s[b] = mfma32(k, qop[b][kk], s[b]);
  }
}

// O^T[128 x 32] += V^T . P^T for one tile and each row block; v_rd = this
// lane's transposing read address. Each V operand feeds every block's hi
// (and lo) MFMA; consecutive MFMAs go to different accumulators.
template <int RB, bool PSPLIT>
__device__ __forceinline__ void pv_tile(f32x16 (&o)[RB][4], const bf16x8 (&ph)[RB][2],
                                        const bf16x8 (&pl)[RB][2], const char* v_rd) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bf16x8 va[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x4 v0 = ds_read_tr(v_rd + (16 * j) * kVRow + 64 * db);
      const bf16x4 v1 = ds_read_tr(v_rd + (16 * j + 8) * kVRow + 64 * db);
      // whole-vector concatenation (element-wise inserts of the transposed
      // halves were mis-lowered by the compiler)
      va[db] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
      for (int db = 0; db < 4; ++db) o[b][db] = mfma32(va[db], ph[b][j], o[b][db]);
    if (PSPLIT) {
#pragma unroll
      for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[b][db] = mfma32(va[db], pl[b][j], o[b][db]);
    }
  }
}

// max over the lane pair (l, l ^ 32) that shares a row: one VALU lane swap
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Keys past `valid` in a partial tile get score -inf (weight 0).
template <bool MASKED>
__device__ __forceinline__ void mask_tile(f32x16& s, int valid, int hl) {
  if (MASKED) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tk = 8 * (i >> 2) + 4 * hl + (i & 3);
      s[i] = tk < valid ? s[i] : kNegInf;
    }
  }
}

// The row's maximum raw score over the tile, times c (both lanes of the row).
__device__ __forceinline__ float tile_max(const f32x16& s, float c) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  return pair_max(mx) * c;
}

// Weights p = 2^(c*s + nm) of one tile, P^T as bf16 (hi + lo with PSPLIT);
// returns this lane's sum of the fp32 weights.
template <bool PSPLIT>
__device__ __forceinline__ float tile_weights(const f32x16& s, float c, float nm, bf16x8 (&ph)[2],
                                              bf16x8 (&pl)[2]) {
  float psum = 0.f;
#pragma unroll
  for (int hj = 0; hj < 2; ++hj) {
    f32x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = fast_exp2(__builtin_fmaf(s[8 * hj + e], c, nm));
      psum += pf[e];
    }
    const bf16x8 hi = __builtin_convertvector(pf, bf16x8);
    ph[hj] = hi;
    if (PSPLIT) pl[hj] = bf16_lo_part(pf, hi);
  }
  return psum;
}

// Issue order for one pipelined tile (one scheduling region): the operand
// reads first, then every MFMA followed by a few VALU instructions of the
// softmax, so the matrix core and the VALU work side by side in one wave.
template <int RB, bool PSPLIT>
__device__ __forceinline__ void tile_schedule() {
  constexpr int kMfma = RB * (PSPLIT ? 24 : 16);
  constexpr int kValuPer = FB_ROWS_VALU_PER;
  __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);        // K operands, V operands (j = 0)
#pragma unroll
  for (int i = 0; i < kMfma; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);
    if (i == 4 * RB) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // V operands (j = 1)
  }
}

// Software pipeline over the key tiles of a chunk, per wave: while the
// VALU runs the softmax of tile t, the matrix core runs S(t+1) = QK(t+1) and
// O += P(t-1).V(t-1). LDS holds eight tile stages (t-1 .. t+5): V(t-1) and
// K(t+1) being read, and tile t+4 being written from the registers loaded
// from global memory two tiles earlier (two register sets, by the parity of
// the tile's position in the chunk).
template <int NW, int RB, int OCC, bool PSPLIT, bool MERGE>
__global__ __launch_bounds__(64 * NW, OCC) void rows_mfma_kernel(RowsParams p) {
  constexpr int RPT = 32 / (NW * 4);              // tile rows staged per thread
  constexpr int kStages = 8;
  constexpr int kSets = 2;                         // register sets: tiles t+4 and t+5
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStage];

  // Work items are (KV group with an unmasked head, chunk, row tile), the
  // groups compacted so that heads a mask skips take no share of the grid.
  // XCD-aware order: workgroup id i runs on XCD i mod 8, and XCD x takes the
  // x-th contiguous range of items, so the row tiles of one (group, chunk)
  // run side by side on one XCD and share its L2 for the K/V tiles.
  const int G = p.group;
  auto group_on = [&](int gg) -> bool {
    if (!p.mask) return true;
    for (int j = 0; j < G; ++j)
      if (p.mask[gg * G + j] == 0) return true;
    return false;
  };
  const int n_on = groups_on(p.mask, p.hkv, G);
  int n_chunks = p.n_chunks;
  int64_t tiles_per_chunk = p.tiles_per_chunk;
  if (p.dyn.on) {
    const RowsSplit sp = rows_dyn_split(n_on, p.dyn);
    n_chunks = sp.chunks;
    tiles_per_chunk = sp.tiles_per_chunk;
  }
  int rt, chunk, g;
  {
    const int n_items = n_on * n_chunks * p.n_rtiles;
    const int id = blockIdx.x;
    const int per = (n_items + 7) >> 3;
    const int item = (id & 7) * per + (id >> 3);
    if ((id >> 3) >= per || item >= n_items) return;
    rt = item % p.n_rtiles;
    const int rest = item / p.n_rtiles;
    chunk = rest % n_chunks;
    int gi = rest / n_chunks;                      // gi-th group that is on
    g = 0;
    for (int gg = 0; gg < p.hkv; ++gg) {
      if (group_on(gg)) {
        if (gi == 0) {
          g = gg;
          break;
        }
        --gi;
      }
    }
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, r32 = lane & 31;
  const int R = p.n_q * G;
  // this lane's row in block b: rows are (query token, query head of the group)
  auto row_of = [&](int b) { return rt * (NW * 32 * RB) + w * (32 * RB) + b * 32 + r32; };

  // Q^T operands: lane holds its row's dims 16 kk + 8 hl .. +8, per block.
  bf16x8 qop[RB][8];
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const int row = row_of(b);
    const bool ok = row < R;
    const int t = ok ? row / G : 0, jh = ok ? row % G : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + static_cast<int64_t>(t) * p.q_st +
                         static_cast<int64_t>(g * G + jh) * p.q_sh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qop[b][kk] = ok ? *reinterpret_cast<const bf16x8*>(qp + 16 * kk + 8 * hl) : bf16x8{};
  }

  const int64_t n_tiles = (p.n_kv + kTile - 1) / kTile;
  const int64_t t_begin = static_cast<int64_t>(chunk) * tiles_per_chunk;
  const int64_t t_end = t_begin + tiles_per_chunk < n_tiles ? t_begin + tiles_per_chunk : n_tiles;
  const int64_t t_last = t_end - 1;                // every launched chunk has a tile

  // staging: thread = (rows lr + 4 NW i of the tile, 16-byte piece lp)
  const int lr = tid >> 4, lp = tid & 15;
  const char* kg = static_cast<const char*>(p.k) + static_cast<int64_t>(g) * p.k_sh * 2;
  const char* vg = static_cast<const char*>(p.v) + static_cast<int64_t>(g) * p.v_sh * 2;
  const int64_t kst = p.k_st * 2, vst = p.v_st * 2;
  const uint32_t koff = static_cast<uint32_t>(lr * kst) + lp * 16;
  const uint32_t voff = static_cast<uint32_t>(lr * vst) + lp * 16;

  // Every step refills the registers unconditionally (tiles past the chunk's
  // last are clamped to it; keys past n_kv to the last key, masked in the
  // scores), so each path through the loop issues the same loads.
  u32x4 kr[kSets][RPT], vr[kSets][RPT];
  auto load = [&](auto set, int64_t tile) {
    constexpr int S = decltype(set)::value;
    tile = tile < t_last ? tile : t_last;
    const int64_t tok0 = tile * kTile;
    if (tok0 + kTile <= p.n_kv) {
      const char* kb = kg + tok0 * kst;
      const char* vb = vg + tok0 * vst;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        kr[S][i] = *reinterpret_cast<const u32x4*>(kb + (4 * NW * i) * kst + koff);
        vr[S][i] = *reinterpret_cast<const u32x4*>(vb + (4 * NW * i) * vst + voff);
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        int64_t tok = tok0 + lr + 4 * NW * i;
        tok = tok < p.n_kv ? tok : p.n_kv - 1;
        kr[S][i] = *reinterpret_cast<const u32x4*>(kg + tok * kst + lp * 16);
        vr[S][i] = *reinterpret_cast<const u32x4*>(vg + tok * vst + lp * 16);
      }
    }
  };
  auto stage_of = [&](int64_t tile) -> char* {
    return lds + (static_cast<int>(tile - t_begin) & (kStages - 1)) * kStage;
  };
  auto store = [&](auto set, int64_t tile) {
    constexpr int S = decltype(set)::value;
    char* kl = stage_of(tile);
    char* vl = kl + kKBytes;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      *reinterpret_cast<u32x4*>(kl + (lr + 4 * NW * i) * kKRow + lp * 16) = kr[S][i];
      *reinterpret_cast<u32x4*>(vl + (lr + 4 * NW * i) * kVRow + lp * 16) = vr[S][i];
    }
  };
  auto valid_of = [&](int64_t tile) -> int {
    const int64_t rem = p.n_kv - tile * kTile;
    return rem < kTile ? static_cast<int>(rem) : kTile;
  };

  // operand addresses within a stage
  const int grp = lane >> 4, s4 = (lane & 15) >> 2, q4 = lane & 3;
  const int k_rd = r32 * kKRow + hl * 16;
  const int v_rd = kKBytes + (4 * (grp >> 1) + s4) * kVRow + 32 * (grp & 1) + 8 * q4;

  f32x16 o[RB][4];
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[b][db] = f32x16{};
  float m_run[RB], l_run[RB];
  bf16x8 ph[RB][2], pl[RB][2];                     // P(t-1); zero before the first tile
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    m_run[b] = kNegInf;
    l_run[b] = 0.f;
    ph[b][0] = ph[b][1] = pl[b][0] = pl[b][1] = bf16x8{};
  }

  // prologue: tiles t_begin, t_begin + 1 staged, t_begin + 2 in registers,
  // the V part of stage (t_begin - 1) zeroed (the first PV adds P = 0 times it)
  // prologue: tiles t_begin .. t_begin + 3 staged, t_begin + 4 and + 5 in
  // the two register sets
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    load(Int<0>{}, t_begin + i);
    store(Int<0>{}, t_begin + i);
  }
  load(Int<0>{}, t_begin + 4);
  load(Int<1>{}, t_begin + 5);
  {
    char* vz = stage_of(t_begin - 1) + kKBytes;
    for (int i = tid; i < kVBytes / 16; i += 64 * NW) *reinterpret_cast<u32x4*>(vz + 16 * i) = u32x4{};
  }
  __syncthreads();
  f32x16 s_cur[RB], s_nxt[RB];
  qk_tile<RB>(stage_of(t_begin) + k_rd, qop, s_cur);

  // one pipelined tile; MASKED only for a partial last tile of the keys.
  // s_in = S(t), computed by the previous tile; s_out receives S(t+1).
  // set: the register set of this tile's position parity; sync: end with
  // the workgroup barrier
  auto iter = [&](int64_t t, auto masked, const f32x16 (&s_in)[RB], f32x16 (&s_out)[RB],
                  auto set, auto sync) {
    constexpr bool M = decltype(masked)::value;
    qk_tile<RB>(stage_of(t + 1) + k_rd, qop, s_out);
    pv_tile<RB, PSPLIT>(o, ph, pl, stage_of(t - 1) + v_rd);
    // The weights take the running max as it stands, so their exponentials
    // do not wait for this tile's max; the max only decides whether the
    // running max must rise (by more than 2^8), and the rare tile where it
    // does recomputes its weights below with the raised max.
    const float c = p.scale_log2;
    f32x16 sm[RB];
    float mx[RB], l_prev[RB];
    bool bump[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      sm[b] = s_in[b];
      mask_tile<M>(sm[b], valid_of(t), hl);
      l_prev[b] = l_run[b];
      l_run[b] = l_prev[b] + tile_weights<PSPLIT>(sm[b], c, m_run[b] == kNegInf ? 0.f : -m_run[b],
                                                  ph[b], pl[b]);
      mx[b] = tile_max(sm[b], c);
      bump[b] = mx[b] > m_run[b] + kRescaleLog2;
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
      asm volatile("" ::"v"(ph[b][0]), "v"(ph[b][1]), "v"(pl[b][0]), "v"(pl[b][1]), "v"(l_run[b]),
                   "v"(mx[b]));
    tile_schedule<RB, PSPLIT>();
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (__any(bump[b])) {
        // raise the max: O (through tile t-1) and l rescaled, this tile's
        // weights recomputed (lanes that keep their max get the same values)
        const float alpha = bump[b] ? fast_exp2(m_run[b] - mx[b]) : 1.f;
        m_run[b] = bump[b] ? mx[b] : m_run[b];
        const float ps = tile_weights<PSPLIT>(sm[b], c, m_run[b] == kNegInf ? 0.f : -m_run[b], ph[b],
                                              pl[b]);
        l_run[b] = l_prev[b] * alpha + ps;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[b][db] *= alpha;
      }
    }
    // eight stages, stores four tiles ahead: a stage read at tile j was
    // written at tile j - 3 (K) or j - 5 (V) and is overwritten at tile
    // j + 5 (K) or j + 3 (V), so one barrier in any three consecutive tiles
    // orders both; the loop syncs after every second tile
    store(set, t + 4);
    load(set, t + 6);
    if (decltype(sync)::value) __syncthreads();
  };
  // two tiles per trip: S alternates between the two register sets
  int64_t tt = t_begin;
  for (; tt + 1 < t_last; tt += 2) {
    iter(tt, Flag<false>{}, s_cur, s_nxt, Int<0>{}, Flag<false>{});
    iter(tt + 1, Flag<false>{}, s_nxt, s_cur, Int<kSets - 1>{}, Flag<true>{});
  }
  if (tt < t_last) {
    iter(tt, Flag<false>{}, s_cur, s_nxt, Int<0>{}, Flag<true>{});
#pragma unroll
    for (int b = 0; b < RB; ++b) s_cur[b] = s_nxt[b];
  }
  // the last tile (position parity picks its register set)
  auto last = [&](auto set) {
    if (valid_of(t_last) < kTile) iter(t_last, Flag<true>{}, s_cur, s_nxt, set, Flag<true>{});
    else iter(t_last, Flag<false>{}, s_cur, s_nxt, set, Flag<true>{});
  };
  if (((t_last - t_begin) & 1) == 0) last(Int<0>{});
  else last(Int<kSets - 1>{});
  pv_tile<RB, PSPLIT>(o, ph, pl, stage_of(t_end - 1) + v_rd);

  // epilogue, per block: lane (r32, hl) holds dims 32 db + 8 q + 4 hl + (0..3) of its row
#pragma unroll
  for (int b = 0; b < RB; ++b) {
    const float l = l_run[b] + __shfl_xor(l_run[b], 32, 64);
    const int row = row_of(b);
    if (row >= R) continue;
    const int t = row / G, h = g * G + row % G;
    if (p.mask && p.mask[h]) continue;
    const int64_t orow_base = static_cast<int64_t>(t) * p.hq + h;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lz = any ? (m_run[b] + __log2f(l)) * kLn2 : kNegInf;
    const f32x16* ob = o[b];
    if (!MERGE) {
      const int64_t orow = static_cast<int64_t>(chunk) * p.out.chunk_stride_rows + orow_base;
      float* a = p.out.a + orow * kD + 4 * hl;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {ob[db][4 * q] * inv, ob[db][4 * q + 1] * inv, ob[db][4 * q + 2] * inv,
                           ob[db][4 * q + 3] * inv};
          *reinterpret_cast<f32x4*>(a + 32 * db + 8 * q) = v;
        }
      if (hl == 0) p.out.l[orow] = lz;
    } else {
      // A_full = (w_out A_out + w_in A_in) / (w_out + w_in), m = max(L_out, L_in)
      const int64_t r = orow_base;
      const float l_prev = p.l_prev[r];
      const float mm = fmaxf(l_prev, lz);
      const float w_out = l_prev == kNegInf ? 0.f : expf(l_prev - mm);
      const float w_in = expf(lz - mm);
      const float den = w_out + w_in;
      const float* ap = p.a_prev + r * kD + 4 * hl;
      float* a = p.out.a + r * kD + 4 * hl;
      float* ai = p.a_raw ? p.a_raw + r * kD + 4 * hl : nullptr;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 vin = {ob[db][4 * q] * inv, ob[db][4 * q + 1] * inv, ob[db][4 * q + 2] * inv,
                             ob[db][4 * q + 3] * inv};
          const f32x4 vp = *reinterpret_cast<const f32x4*>(ap + 32 * db + 8 * q);
          f32x4 vf;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vf[e] = w_out == 0.f ? vin[e] : (w_out * vp[e] + w_in * vin[e]) / den;
          *reinterpret_cast<f32x4*>(a + 32 * db + 8 * q) = vf;
          if (ai) *reinterpret_cast<f32x4*>(ai + 32 * db + 8 * q) = vin;
        }
      if (hl == 0) {
        if (p.out.l) p.out.l[r] = mm + logf(den);
        if (p.l_raw) p.l_raw[r] = lz;
      }
    }
  }
}

}  // namespace

int rows_tile_rows() { return FB_ROWS_WAVES * 32 * FB_ROWS_BLOCKS; }
int rows_occupancy() { return FB_ROWS_OCC; }

hipError_t launch_rows(const RowsParams& p, hipStream_t s) {
  const int per = (p.n_items + 7) / 8;
  const dim3 grid(per * 8);
  if (p.a_prev)
    hipLaunchKernelGGL((rows_mfma_kernel<FB_ROWS_WAVES, FB_ROWS_BLOCKS, FB_ROWS_OCC, FB_ROWS_PSPLIT != 0, true>),
                       grid, dim3(64 * FB_ROWS_WAVES), 0, s, p);
  else
    hipLaunchKernelGGL((rows_mfma_kernel<FB_ROWS_WAVES, FB_ROWS_BLOCKS, FB_ROWS_OCC, FB_ROWS_PSPLIT != 0, false>),
                       grid, dim3(64 * FB_ROWS_WAVES), 0, s, p);
  return hipGetLastError();
}

}  // namespace fb
