// Same-step chunk attention on CDNA4 (gfx950): a flash-style kernel with
// bf16 MFMA for both products and an fp32 online softmax.
//
// What it computes ("PhysisServe -- Wan2.2 5B" model card, "Inference
// profile"): for every head and query, softmax(scale * q K_win^T) V_win over
// the window [sink | same-step ring window | own chunk], no mask.  The
// window is not concatenated: it arrives as up to three runs of keys (the
// sink, then up to two runs of ring slots) and every 16-byte piece of a tile
// is fetched from the run that holds it.
//
// Tiling.  A workgroup is 4 waves; each wave owns 32 query rows of one head
// (128 rows per workgroup).  Keys stream through LDS in tiles of 64: K rows
// [64][d] and V^T rows [d][64], unpadded, with the 16-byte chunks of every
// row XOR-swizzled so that the MFMA operand reads (16 lanes on 16
// consecutive rows, one logical chunk) hit 16 distinct bank groups.  Tiles
// are fetched straight into LDS (global_load_lds_dwordx4, no staging
// registers): each lane is given the global 16-byte piece that belongs at
// its LDS position, so the swizzle and the permuted K-row order cost
// nothing, and every wave issues the same number of fetches.  Two LDS
// buffers alternate; tile t+1 is in flight while tile t is computed, with
// one barrier per tile.
//
// Products use v_mfma_f32_32x32x16_bf16 (32x32 output blocks; the matrix
// units run it at the same FLOP rate as the 16x16x32 form, and a wave's
// operand bytes depend on its tile, not on the form, but its accumulator
// layout gives a lane 16 scores of a single query, so the softmax needs only
// a two-lane reduction and the weights go from registers straight into the
// B operand of the PV product): per tile and wave
//   S^T[64 keys x 32 queries] = K_tile Q^T      2 blocks x d/16 steps
//   O^T[d x 32 queries]      += V^T_tile P^T    d/32 blocks x 4 steps
// With the queries as the N columns, lane l holds the scores of query l % 32
// for 32 of the tile's 64 keys (lanes l and l + 32 share a query).  K rows
// sit in LDS in a permuted order (bits 2 and 3 of the row index swapped) so
// that the 8 consecutive scores a lane holds for each 16-key step of the PV
// product are 8 consecutive keys: P goes from registers straight into the B
// operand.
//
// Softmax.  Scores stay raw; the scale (times log2 e) is folded into one FMA
// per score before exp2.  A tile is taken as two 32-key blocks so that one
// block's softmax runs on the vector ALUs while the matrix units work on the
// other: S^T of block 1 is issued before block 0's weights, and block 0's
// PV steps before block 1's weights (scheduling-group barriers interleave
// them).  The running max is lazy, per block: a block's weights are computed
// against the stale max and kept as long as each lane's sum of them stays
// <= 2^8 (then no weight exceeds 2^8, which bf16 and the fp32 accumulators
// hold exactly enough); only when that sum is larger, NaN or infinite (rare;
// always on a split's first block, where the max is -inf) is the block's
// 2-lane max taken, O and the running sums rescaled and the block's weights
// recomputed.  The check needs no max over the scores of every block.  The
// row sums add the same bf16-rounded P that multiplies V (v_dot2_f32_bf16
// against ones), so numerator and denominator see the same weights.  Only
// the last tile of a split can be partial; it runs after the loop with a
// masked copy of the tile code, so the loop carries one copy.
//
// Occupancy.  880 queries x 24 heads is only 168 workgroups of 128 rows for
// 256 CUs (21 for a 3-head share), so the key range is split into as many
// parts as fill the chip's workgroup slots once (3 and 24 parts there); each
// part writes normalised fp16 partials and a float32 log2-domain log-sum-exp,
// and a second kernel merges them in float32 (softmax over a concatenation
// equals the LSE-weighted merge of per-part softmaxes).
//
// L2 locality.  Workgroups are dispatched round-robin over the 8 XCDs, each
// with its own L2.  The block -> work-unit map gives every XCD a contiguous
// run of units ordered (head, split)-major, so the query tiles that read the
// same K/V run on the same XCD at the same time.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ckv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int QT = kAttnQueryTile;  // 128
constexpr int KT = kAttnKeyTile;    // 64
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;
constexpr float kTileSumLimit = 256.0f;  // lazy rescale: a lane's tile sum of weights at most 2^8
static_assert(KT == 64, "a key tile is two 32-key blocks");
constexpr int KS = KT / 16;           // 16-key steps of the PV product per tile
// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

template <int D>
struct Tile {
  static constexpr int kChunksK = D / 8;              // 16-byte chunks per K row
  static constexpr int kRowBytesK = 2 * D;
  static constexpr int kRowBytesV = 2 * KT;           // 128: 8 chunks per V^T row
  static constexpr int kBytesK = KT * kRowBytesK;
  static constexpr int kBytesV = D * kRowBytesV;
  static constexpr int kBlocksK = kBytesK / 1024;     // 1 KB blocks, one wave instruction each
  static constexpr int kBlocksV = kBytesV / 1024;
  static constexpr int kSlotsK = kBlocksK / kWaves;   // fetch instructions per wave per tile
  static constexpr int kSlotsV = kBlocksV / kWaves;
  static_assert(kBlocksK % kWaves == 0 && kBlocksV % kWaves == 0, "tiles split evenly over the waves");
};

// XOR swizzle of the 16-byte chunks of LDS row r.  Rows of 16 chunks (K at
// d = 128) use r mod 16; rows of 8 chunks (V^T, and K at d = 64) use
// (r / 2) mod 8: two such rows fill the 64 banks once, so rows 2m and 2m+1
// differ in bank half and rows with different m in chunk.
template <int Chunks>
__device__ inline int swz(int r) {
  return Chunks == 16 ? (r & 15) : ((r >> 1) & 7);
}

// K rows sit in LDS in a permuted order: LDS row p holds tile key p with
// bits 2 and 3 swapped.  S^T block mb then gives lane l (h = l / 32) the
// scores of LDS rows 32mb + 8g + 4h + e (g, e = 0..3), i.e. of tile keys
// 32mb + 16(g/2) + 8h + 4(g%2) + e: for PV step ks = 2mb + g/2 its eight
// scores 8(g/2) .. 8(g/2)+7 are keys 16ks + 8h .. 16ks + 8h + 7, the B
// operand's k-range for that lane.
__device__ inline int key_of_lds_row(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

__device__ inline bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// Max and sum of x over the lane pair l, l ^ 32 that shares a query.  After
// the swap one result holds x[l] and the other x[l ^ 32] in every lane (in
// either order), so both lanes compute the same value bit for bit.
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max of two / three floats, as compiler builtins: the scores they read come
// straight from MFMA accumulators, and only instructions the compiler can see
// get the wait states a VALU read of an MFMA result needs (an inline-asm max
// here read accumulators that were still being written).
__device__ inline float max3f(float a, float b, float c) { return __builtin_fmaxf(a, __builtin_fmaxf(b, c)); }
__device__ inline float max2f(float a, float b) { return __builtin_fmaxf(a, b); }

// The up to three runs of this head's window, loaded once into uniform
// scalars (no indexed access to the parameter block, which would force a
// private-memory copy of it).
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline const char* uni(const void* ptr) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(ptr);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

struct Runs {
  const char *k0, *k1, *k2;  // this head's K row of each run's first key
  const char *v0, *v1, *v2;  // this head's V^T column of each run's first key
  int vrs0, vrs1, vrs2;      // V^T row strides (elements)
  int e0, e1, e2;            // cumulative key ends of the runs
};

__device__ inline Runs load_runs(const AttnParams& p, int head) {
  Runs R;
  R.k0 = uni(p.k[0] + head * p.k_head_stride[0]);
  R.k1 = uni(p.k[1] + head * p.k_head_stride[1]);
  R.k2 = uni(p.k[2] + head * p.k_head_stride[2]);
  R.v0 = uni(p.vt[0] + head * p.vt_head_stride[0]);
  R.v1 = uni(p.vt[1] + head * p.vt_head_stride[1]);
  R.v2 = uni(p.vt[2] + head * p.vt_head_stride[2]);
  R.vrs0 = uni(p.vt_row_stride[0]);
  R.vrs1 = uni(p.vt_row_stride[1]);
  R.vrs2 = uni(p.vt_row_stride[2]);
  R.e0 = uni(p.seg_end[0]);
  R.e1 = uni(p.seg_end[1]);
  R.e2 = uni(p.seg_end[2]);
  return R;
}

// The piece lane l fetches for slot i of wave w: block b = w + 4i of the
// tile, i.e. LDS byte 1024 b + 16 l = LDS row r, physical chunk pc; it holds
// logical chunk pc ^ swz(r) of that row.
template <int D>
__device__ inline int k_piece_row(int w, int l, int i) {
  return (w + kWaves * i) * (1024 / Tile<D>::kRowBytesK) + l / Tile<D>::kChunksK;
}
template <int D>
__device__ inline int k_piece_chunk(int w, int l, int i) {
  return (l % Tile<D>::kChunksK) ^ swz<Tile<D>::kChunksK>(k_piece_row<D>(w, l, i));
}
__device__ inline int v_piece_row(int w, int l, int i) { return (w + kWaves * i) * 8 + l / 8; }
__device__ inline int v_piece_chunk(int w, int l, int i) { return (l % 8) ^ swz<8>(v_piece_row(w, l, i)); }

// Per-lane byte offsets of this lane's pieces from a tile's first key in a
// run; unsigned, so each fetch is a scalar base plus a 32-bit lane offset.
template <int D>
struct LaneSlots {
  unsigned k_off[Tile<D>::kSlotsK];  // (key * d + 8 * chunk) * 2
  unsigned v_off[Tile<D>::kSlotsV];  // (dim * row_stride + 8 * chunk) * 2 in the current run
};

// Hide a per-lane value from the optimiser, so that nothing computed from it
// is hoisted above this point (keeps the rare straddling path's address terms
// out of the registers of the key loop).
template <class T>
__device__ inline void opaque(T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// One 16-byte-per-lane global -> LDS transfer (lane l lands at lds + 16 l).
// The host pass of a HIP compile cannot resolve this builtin inside nested
// device templates; only the device pass needs the body.
__device__ inline void lds_dma16(const void* src, lds_void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

// Sequential walk over this workgroup's keys.  The run (sink area or a run
// of ring slots) holding the next tile changes at most twice per workgroup;
// within a run a tile's source is a uniform base plus fixed per-lane offsets.
// Runs are chosen by comparing key boundaries, never by an index (an index
// would turn the choice into a table in private memory).
struct RunCursor {
  int begin, end;  // key range of the current run
  const char* k;   // K row of key `begin`
  const char* vt;  // V^T column of key `begin`
};

template <int D>
__device__ inline void cursor_set(RunCursor& c, LaneSlots<D>& s, int w, int l, int begin, int end, const char* k,
                                  const char* vt, int vrs) {
  c.begin = begin;
  c.end = end;
  c.k = k;
  c.vt = vt;
#pragma unroll
  for (int i = 0; i < Tile<D>::kSlotsV; ++i)
    s.v_off[i] = (unsigned)(v_piece_row(w, l, i) * vrs + 8 * v_piece_chunk(w, l, i)) * 2u;
}

// Place the cursor on the run holding key j (uniform j).
template <int D>
__device__ inline void cursor_seek(const Runs& R, RunCursor& c, LaneSlots<D>& s, int w, int l, int j) {
  if (j < R.e0)
    cursor_set<D>(c, s, w, l, 0, R.e0, R.k0, R.v0, R.vrs0);
  else if (j < R.e1)
    cursor_set<D>(c, s, w, l, R.e0, R.e1, R.k1, R.v1, R.vrs1);
  else
    cursor_set<D>(c, s, w, l, R.e1, R.e2, R.k2, R.v2, R.vrs2);
}

// Source of key j's K row / of V^T row `dim` at key j, for per-lane j.
template <int D>
__device__ inline const char* k_row_of(const Runs& R, int j) {
  return j < R.e0 ? R.k0 + (long long)j * (2 * D)
                  : (j < R.e1 ? R.k1 + (long long)(j - R.e0) * (2 * D) : R.k2 + (long long)(j - R.e1) * (2 * D));
}
__device__ inline const char* vt_at(const Runs& R, int dim, int j) {
  return j < R.e0 ? R.v0 + ((long long)dim * R.vrs0 + j) * 2
                  : (j < R.e1 ? R.v1 + ((long long)dim * R.vrs1 + (j - R.e0)) * 2
                              : R.v2 + ((long long)dim * R.vrs2 + (j - R.e1)) * 2);
}

// Enqueue the fetch of key tile [t0, t0 + KT) into one LDS buffer pair.
template <int D>
__device__ inline void fetch_tile(const Runs& R, LaneSlots<D>& s, RunCursor& c, int w, int l, int t0, int key_begin,
                                  int key_end, char* sk, char* sv) {
  using T = Tile<D>;
  if (t0 >= c.end) cursor_seek<D>(R, c, s, w, l, t0);
  if (t0 + KT <= c.end && t0 + KT <= key_end) {
    // uniform bases made explicit (readfirstlane) so that each fetch stays
    // scalar base + 32-bit lane offset
    const char* kb = uni(c.k + (long long)(t0 - c.begin) * (2 * D));
    const char* vb = uni(c.vt + (long long)(t0 - c.begin) * 2);
    // (the offsets pass through opaque() so that their 64-bit extension is
    // not hoisted out of the key loop, where it would double their registers)
#pragma unroll
    for (int i = 0; i < T::kSlotsK; ++i) {
      unsigned off = s.k_off[i];
      opaque(off);
      lds_dma16(kb + off, (lds_void*)(sk + (w + kWaves * i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < T::kSlotsV; ++i) {
      unsigned off = s.v_off[i];
      opaque(off);
      lds_dma16(vb + off, (lds_void*)(sv + (w + kWaves * i) * 1024));
    }
  } else {
    // Tile straddles two runs or the end of this split's keys: per-lane
    // lookup; keys past the end fetch key_begin (finite data; masked later).
    opaque(l);
#pragma unroll
    for (int i = 0; i < T::kSlotsK; ++i) {
      int j = t0 + key_of_lds_row(k_piece_row<D>(w, l, i));
      if (j >= key_end) j = key_begin;
      lds_dma16(k_row_of<D>(R, j) + 16 * k_piece_chunk<D>(w, l, i), (lds_void*)(sk + (w + kWaves * i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < T::kSlotsV; ++i) {
      int j = t0 + 8 * v_piece_chunk(w, l, i);  // runs are multiples of 8 keys: a piece never straddles two runs
      if (j >= key_end) j = key_begin;
      lds_dma16(vt_at(R, v_piece_row(w, l, i), j), (lds_void*)(sv + (w + kWaves * i) * 1024));
    }
  }
}

constexpr int kSchedValu = 0x002;

// P = 2^(s * scale_log2 - m) in bf16 for one 32-key block (the B operands of
// its two 16-key PV steps); returns this lane's sum of the same bf16 weights.
__device__ inline float block_weights(const f32x16& s, bf16x8& p0, bf16x8& p1, float m, float scale_log2) {
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  const float neg_m = -m;
  float ts = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, neg_m));
    const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r + 1], scale_log2, neg_m));
    const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
    ts = __builtin_amdgcn_fdot2_f32_bf16(pk, one2, ts, false);
    if (r < 8) {
      p0[r] = pk[0];
      p0[r + 1] = pk[1];
    } else {
      p1[r - 8] = pk[0];
      p1[r - 7] = pk[1];
    }
  }
  return ts;
}

// Rare path of the lazy rescale: raise m to the block's 2-lane max (log2
// domain) and rescale O and the running sum to it.
template <int DB>
__device__ inline void rescale_to_block(const f32x16& s, f32x16 (&o)[DB], float& m, float& lsum, float scale_log2) {
  float b0 = max3f(s[0], s[1], s[2]);
  float b1 = max3f(s[3], s[4], s[5]);
  float b2 = max3f(s[6], s[7], s[8]);
  float b3 = max3f(s[9], s[10], s[11]);
  float b4 = max3f(s[12], s[13], s[14]);
  b0 = max3f(b0, b1, s[15]);
  b2 = max3f(b2, b3, b4);
  const float m_new = fmaxf(m, pair_max(max2f(b0, b2)) * scale_log2);
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);
  lsum *= alpha;
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] *= alpha;
  m = m_new;
}

// One key tile for a wave's 32 queries:
//   S^T = K_tile Q^T, online softmax per query, O^T += V^T_tile P^T,
// taken as two 32-key blocks so that each block's softmax runs while the
// matrix units work on the other: S^T of block 1 is issued before the
// weights of block 0 are computed, and the PV steps of block 0 before the
// weights of block 1.  Each block has its own lazy-rescale check.
// S value [r] of block mb is the score of tile key 32mb + 16(r/8) + 8h +
// 4((r/4)%2) + r%4 (h = lane / 32) for query lane % 32.  O value (db)[r] is
// head dim 32db + 8(r/4) + 4h + r%4 of that query.  ka[kk] / va[ks] are this
// lane's operand byte offsets within a K / V^T tile for 16-dim step kk /
// 16-key step ks.
template <int D, bool kMasked>
__device__ inline void attend_tile(const char* sk, const char* sv, const int (&ka)[D / 16], const int (&va)[KS],
                                   const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32], float& m, float& lsum,
                                   float scale_log2, int t0, int key_end, int h) {
  using T = Tile<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int kWeightValu = 48 / KK;  // VALU of one block's weights per MFMA it hides behind
  f32x16 s0, s1;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = 0.f;
    s1[r] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sk + ka[kk]));
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s0, 0, 0, 0);
  }
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sk + 32 * T::kRowBytesK + ka[kk]));
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s1, 0, 0, 0);
  }
  if (kMasked) {
    // keys of this lane's scores past key_end get -inf; the bound is formed
    // here and hidden from the optimiser so that nothing per score is hoisted
    // out of the key loop
    int lim = key_end - t0 - 8 * h;
    opaque(lim);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k0 = 16 * (r / 8) + 4 * ((r / 4) % 2) + r % 4;
      if (k0 >= lim) s0[r] = -INFINITY;
      if (k0 + 32 >= lim) s1[r] = -INFINITY;
    }
  }
  bf16x8 pf[KS];
  float ts = block_weights(s0, pf[0], pf[1], m, scale_log2);
  // K operand reads 4 ahead of their MFMAs; block 0's weights between block
  // 1's MFMAs
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (j < KK - 4) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, kWeightValu, 0);
  }
  // Lazy rescale: the weights are kept while this lane's sum of them stays
  // <= 2^8, so every weight is <= 2^8, which bf16 and the float32
  // accumulators hold exactly enough.  Otherwise (rarely; always on a
  // split's first block, where m = -inf makes the sum NaN or inf) O and the
  // running sum are rescaled to the block's max and the weights recomputed.
  if (__any(!(ts <= kTileSumLimit))) {
    rescale_to_block<DB>(s0, o, m, lsum, scale_log2);
    ts = block_weights(s0, pf[0], pf[1], m, scale_log2);
  }
  lsum += ts;

  // PV steps of block 0, block 1's weights between them; block 1's V^T
  // operands are read here too, so that its PV steps after the check issue
  // without waiting for LDS
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sv + db * 32 * T::kRowBytesV + va[ks]));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
    }
  bf16x8 vb[2][DB];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      vb[ks][db] = as_bf16x8(*reinterpret_cast<const uint4*>(sv + db * 32 * T::kRowBytesV + va[2 + ks]));
  ts = block_weights(s1, pf[2], pf[3], m, scale_log2);
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
  for (int j = 0; j < 2 * DB; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
    // the other 4 DB - 4 operand reads, two after each MFMA while they last
    if (4 * DB - 4 - 2 * j >= 2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    else if (4 * DB - 4 - 2 * j == 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
    __builtin_amdgcn_sched_group_barrier(kSchedValu, 48 / (2 * DB), 1);
  }
  if (__any(!(ts <= kTileSumLimit))) {
    rescale_to_block<DB>(s1, o, m, lsum, scale_log2);
    ts = block_weights(s1, pf[2], pf[3], m, scale_log2);
  }
  lsum += ts;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[ks][db], pf[2 + ks], o[db], 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void chunk_attn_kernel(AttnParams p) {
  using T = Tile<D>;
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char sk0[T::kBytesK], sk1[T::kBytesK];
  __shared__ __attribute__((aligned(1024))) char sv0[T::kBytesV], sv1[T::kBytesV];

  // Work unit: contiguous runs of (head, split, q-tile) per XCD.
  const int units = p.q_tiles * p.num_heads * p.n_splits;
  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int per = units / kXcds, extra = units % kXcds;
  const int unit = xcd * per + (xcd < extra ? xcd : extra) + li;
  const int qt = unit % p.q_tiles;
  const int grp = unit / p.q_tiles;
  const int split = grp % p.n_splits;
  const int head = grp / p.n_splits;

  const int key_begin = (int)((long long)p.key_tiles * split / p.n_splits) * KT;
  const int key_end = min((int)((long long)p.key_tiles * (split + 1) / p.n_splits) * KT, p.n_keys);
  const int t_begin = key_begin / KT, t_end = (key_end + KT - 1) / KT;

  // wave index as a scalar: block choices and LDS-DMA bases depend on it
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int h = lane / 32, c32 = lane % 32;
  int ka[KK], va[KS];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ka[kk] = c32 * T::kRowBytesK + 16 * ((2 * kk + h) ^ swz<T::kChunksK>(c32));
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) va[ks] = c32 * T::kRowBytesV + 16 * ((2 * ks + h) ^ swz<8>(c32));

  LaneSlots<D> slots;
#pragma unroll
  for (int i = 0; i < T::kSlotsK; ++i)
    slots.k_off[i] =
        (unsigned)(key_of_lds_row(k_piece_row<D>(wave, lane, i)) * D + 8 * k_piece_chunk<D>(wave, lane, i)) * 2u;
  const Runs runs = load_runs(p, head);
  RunCursor cursor;
  cursor_seek<D>(runs, cursor, slots, wave, lane, key_begin);

  // Q^T B operand: lane holds head dims 16kk + 8h .. +8 of query c32.
  const int q_row = qt * QT + wave * 32 + c32;
  const bool q_ok = q_row < p.n_queries;
  bf16x8 qf[KK];
  {
    const uint16_t* qp = p.q + ((long long)(q_ok ? q_row : 0) * p.num_heads + head) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = as_bf16x8(q_ok ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0));
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY;    // running max of scaled scores (log2 domain)
  float lsum = 0.f;       // this lane's share of the running sum

  fetch_tile<D>(runs, slots, cursor, wave, lane, t_begin * KT, key_begin, key_end, sk0, sv0);
  // Tiles [t_begin, t_full) are whole: they run in pairs (buffer 0, then
  // buffer 1), then a last whole tile if their count is odd; a partial last
  // tile (keys up to key_end) runs after them with the masked copy of the
  // tile code, in the buffer its parity gives.
  const int t_full = min(key_end / KT, t_end);
  int t = t_begin;
  for (; t + 1 < t_full; t += 2) {
    // buffer 0 holds tile t; tile t+1 goes to buffer 1 while t is computed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    fetch_tile<D>(runs, slots, cursor, wave, lane, (t + 1) * KT, key_begin, key_end, sk1, sv1);
    attend_tile<D, false>(sk0, sv0, ka, va, qf, o, m, lsum, p.scale_log2, t * KT, key_end, h);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < t_end) fetch_tile<D>(runs, slots, cursor, wave, lane, (t + 2) * KT, key_begin, key_end, sk0, sv0);
    attend_tile<D, false>(sk1, sv1, ka, va, qf, o, m, lsum, p.scale_log2, (t + 1) * KT, key_end, h);
  }
  if (t < t_full) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < t_end) fetch_tile<D>(runs, slots, cursor, wave, lane, (t + 1) * KT, key_begin, key_end, sk1, sv1);
    attend_tile<D, false>(sk0, sv0, ka, va, qf, o, m, lsum, p.scale_log2, t * KT, key_end, h);
    ++t;
  }
  if (t < t_end) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const bool odd = ((t - t_begin) & 1) != 0;
    attend_tile<D, true>(odd ? sk1 : sk0, odd ? sv1 : sv0, ka, va, qf, o, m, lsum, p.scale_log2, t * KT, key_end, h);
  }

  const float ltot = pair_sum(lsum);
  const float inv = 1.f / ltot;
  if (!q_ok) return;
  // lane holds dims 32db + 8g + 4h + (0..3) for g = 0..3
  if (p.n_splits == 1) {
    uint16_t* op = p.out + ((long long)q_row * p.num_heads + head) * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 lo = {(__bf16)(o[db][4 * g] * inv), (__bf16)(o[db][4 * g + 1] * inv)};
        const bf16x2 hi = {(__bf16)(o[db][4 * g + 2] * inv), (__bf16)(o[db][4 * g + 3] * inv)};
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * g) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
  } else {
    const long long row = ((long long)split * p.n_queries + q_row) * p.num_heads + head;
    uint16_t* op = p.part_o + row * D + 4 * h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // normalised partials (|o| <= max |v|) in fp16: 11 significant bits
        const half2 lo = {(_Float16)(o[db][4 * g] * inv), (_Float16)(o[db][4 * g + 1] * inv)};
        const half2 hi = {(_Float16)(o[db][4 * g + 2] * inv), (_Float16)(o[db][4 * g + 3] * inv)};
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * g) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    if (h == 0) p.part_lse[row] = m + __log2f(ltot);
  }
}

// Merge of the key splits: O = sum_j 2^(lse_j - M) O_j / sum_j 2^(lse_j - M),
// M = max_j lse_j.  G adjacent lanes share 8 dims (16 bytes of each fp16
// partial) of one (query, head) row; lane g of the group takes splits g,
// g + G, g + 2G, ... (MaxSplits / G of them), loading every one's
// log-sum-exp and partial before it uses any, so a row costs two memory round
// trips whatever the split count.  The group then takes its max of the
// log-sum-exps and its sums with lane shuffles (a fixed order, so repeated
// calls agree bit for bit), and lane 0 stores.  Many splits (few heads) get
// G = 4: four times the threads of one lane per 8 dims, which would leave
// most CUs idle at 3 heads.
template <int D, int MaxSplits, int G>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  constexpr int TPR = D / 8;          // 16-byte pieces per (query, head) row
  constexpr int PER = MaxSplits / G;  // splits per lane
  static_assert(MaxSplits % G == 0 && 256 % (TPR * G) == 0, "groups tile the block");
  const long long rows = (long long)p.n_queries * p.num_heads;
  const int g = threadIdx.x % G;
  const int c8 = (threadIdx.x / G) % TPR;
  const long long row = (long long)blockIdx.x * (256 / (TPR * G)) + threadIdx.x / (TPR * G);
  if (row >= rows) return;  // uniform over each group of G lanes (same row)
  float lse[PER];
  uint4 part[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = g + G * i;
    lse[i] = j < p.n_splits ? p.part_lse[j * rows + row] : -INFINITY;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = g + G * i;
    part[i] = j < p.n_splits ? *reinterpret_cast<const uint4*>(p.part_o + (j * rows + row) * D + 8 * c8)
                             : make_uint4(0, 0, 0, 0);
  }
  float mx = lse[0];
#pragma unroll
  for (int i = 1; i < PER; ++i) mx = fmaxf(mx, lse[i]);
#pragma unroll
  for (int off = 1; off < G; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  float wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float w = g + G * i < p.n_splits ? __builtin_amdgcn_exp2f(lse[i] - mx) : 0.f;
    wsum += w;
    const uint32_t words[4] = {part[i].x, part[i].y, part[i].z, part[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const half2 v = __builtin_bit_cast(half2, words[e]);
      acc[2 * e] += w * (float)v[0];
      acc[2 * e + 1] += w * (float)v[1];
    }
  }
#pragma unroll
  for (int off = 1; off < G; off <<= 1) {
    wsum += __shfl_xor(wsum, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (g != 0) return;
  const float inv = 1.f / wsum;
  uint32_t packed[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16x2 b = {(__bf16)(acc[2 * e] * inv), (__bf16)(acc[2 * e + 1] * inv)};
    packed[e] = __builtin_bit_cast(uint32_t, b);
  }
  *reinterpret_cast<uint4*>(p.out + row * D + 8 * c8) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

template <int D, int MaxSplits, int G>
void launch_combine_with(const AttnParams& p, hipStream_t s) {
  const int blocks = (int)(((long long)p.n_queries * p.num_heads * (D / 8) * G + 255) / 256);
  hipLaunchKernelGGL((attn_combine_kernel<D, MaxSplits, G>), dim3(blocks), dim3(256), 0, s, p);
}

template <int D>
void launch_combine(const AttnParams& p, hipStream_t s) {
  if (p.n_splits <= 4)
    launch_combine_with<D, 4, 1>(p, s);
  else if (p.n_splits <= 8)
    launch_combine_with<D, 8, 2>(p, s);
  else
    launch_combine_with<D, kAttnMaxSplits, 4>(p, s);
}

}  // namespace

hipError_t launch_chunk_attention(const AttnParams& p, int head_dim, hipStream_t s) {
  if (p.n_queries <= 0 || p.n_keys <= 0 || p.n_splits < 1 || p.n_splits > kAttnMaxSplits) return hipErrorInvalidValue;
  const int units = p.q_tiles * p.num_heads * p.n_splits;
  if (head_dim == 128) {
    hipLaunchKernelGGL(chunk_attn_kernel<128>, dim3(units), dim3(kThreads), 0, s, p);
    if (p.n_splits > 1) launch_combine<128>(p, s);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(chunk_attn_kernel<64>, dim3(units), dim3(kThreads), 0, s, p);
    if (p.n_splits > 1) launch_combine<64>(p, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ckv
