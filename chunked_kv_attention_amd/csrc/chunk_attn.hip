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
// Products use v_mfma_f32_16x16x32_bf16 (16x16 output blocks): per tile and
// wave
//   S^T[64 keys x 32 queries] = K_tile Q^T      8 independent 16x16 blocks
//   O^T[d x 32 queries]      += V^T_tile P^T    2d/16 independent blocks
// so both products keep many accumulation chains in flight.  With the
// queries as the N columns, a lane holds 16 scores of each of its 2 queries;
// a query's row max needs a 4-lane exchange (lane xor 16, xor 32).  K rows
// sit in LDS in a permuted order chosen so that the 8 scores a lane holds
// for each 32-key step of the PV product are 8 consecutive keys, so P goes
// from registers straight into the B operand.
//
// Softmax.  Scores stay raw; the scale (times log2 e) is folded into one FMA
// per score before exp2.  The running max is lazy: O and the running sums are
// rescaled only when a tile raises some row's max by more than 2^8 (a
// wave-uniform branch), otherwise the stale max is kept and P may reach 256,
// which bf16 and the fp32 accumulators hold exactly enough.  The test needs
// no cross-lane max: each lane compares its own raw scores of a query with
// that query's threshold (m + 8) / (scale log2 e), and the 4-lane max is
// taken only inside the rare rescale branch.  The row sums add the same
// bf16-rounded P that multiplies V (v_dot2_f32_bf16 against ones), so
// numerator and denominator see the same weights.
//
// Occupancy.  880 queries x 24 heads is only 168 workgroups of 128 rows for
// 256 CUs, so the key range is split into up to 4 parts when that fills the
// chip better; each part writes normalised fp32 partials and a log2-domain
// log-sum-exp, and a second kernel merges them (softmax over a concatenation
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int QT = kAttnQueryTile;  // 128
constexpr int KT = kAttnKeyTile;    // 64
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int KB = KT / 16;           // 16-key blocks of S^T per tile
constexpr int KS = KT / 32;           // 32-key steps of the PV product per tile
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

// K rows sit in LDS in a permuted order: LDS row p = 32s + 16b + 4h + i holds
// tile key 32s + 8h + 4b + i.  MFMA block kb = 2s + b then reads LDS rows
// 16kb .. 16kb+15, and the lane group h gets keys 32s + 8h + 4b + (0..3).
__device__ inline int key_of_lds_row(int p) { return (p & ~31) | (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3); }

__device__ inline bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// max over the 4 lanes l, l^16, l^32, l^48 that share a query
__device__ inline float quad_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// max of finite floats without the quieting of NaN inputs that fmaxf implies
__device__ inline float max3f(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(a, fmaxf(b, c));
#endif
}
__device__ inline float max2f(float a, float b) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
#else
  return fmaxf(a, b);
#endif
}

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

// One key tile for a wave's 32 queries (2 blocks of 16):
//   S^T = K_tile Q^T, online softmax per query, O^T += V^T_tile P^T.
// S value (kb, qb)[i] is the score of tile key 32s + 8h + 4b + i (kb = 2s + b,
// h = lane / 16) for query 16qb + lane % 16.  O value (db, qb)[i] is head dim
// 16db + 4h + i of that query.  ka[kk] / va[ks] are this lane's operand byte
// offsets within a K / V^T tile for 32-dim step kk / 32-key step ks.
template <int D>
__device__ inline void attend_tile(const char* sk, const char* sv, const int (&ka)[D / 32], const int (&va)[KS],
                                   const bf16x8 (&qf)[D / 32][2], f32x4 (&o)[D / 16][2], float (&m)[2],
                                   float (&thr)[2], float (&lsum)[2], float scale_log2, bool masked, int t0, int key_end, int h) {
  using T = Tile<D>;
  constexpr int KK = D / 32;
  constexpr int DB = D / 16;
  f32x4 s[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sk + kb * 16 * T::kRowBytesK + ka[kk]));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[kk][qb], s[kb][qb], 0, 0, 0);
    }

  // Keep the K operand reads 4 groups ahead of the MFMAs that consume them
  // (LDS latency spans several 16-cycle MFMAs).
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
  for (int j = 0; j < KB * KK - 4; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (t0 + 32 * (kb / 2) + 8 * h + 4 * (kb % 2) + i >= key_end) s[kb][qb][i] = -INFINITY;
  }
  // Rescale test without the cross-lane max: a query needs a new max only if
  // one of its raw scores exceeds thr = (m + 2^8 headroom) / scale_log2, and
  // every lane can test its own 16 scores of each query.  The 4-lane max is
  // taken only in the rare branch.
  float lm[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float a = max3f(s[0][qb][0], s[0][qb][1], s[0][qb][2]);
    float b = max3f(s[0][qb][3], s[1][qb][0], s[1][qb][1]);
    float c = max3f(s[1][qb][2], s[1][qb][3], s[2][qb][0]);
    float d = max3f(s[2][qb][1], s[2][qb][2], s[2][qb][3]);
    float e = max3f(s[3][qb][0], s[3][qb][1], s[3][qb][2]);
    a = max3f(a, b, s[3][qb][3]);
    c = max3f(c, d, e);
    lm[qb] = max2f(a, c);
  }
  if (__any(lm[0] > thr[0] || lm[1] > thr[1])) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_new = fmaxf(m[qb], quad_max(lm[qb]) * scale_log2);
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - m_new);
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db][qb] *= alpha;
      m[qb] = m_new;
      thr[qb] = (m_new + kRescaleLog2) / scale_log2;
    }
  }

  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 pf[KS][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float neg_m = -m[qb];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], scale_log2, neg_m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i + 1], scale_log2, neg_m));
        const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
        lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(pk, one2, lsum[qb], false);
        pf[kb / 2][qb][4 * (kb % 2) + i] = pk[0];
        pf[kb / 2][qb][4 * (kb % 2) + i + 1] = pk[1];
      }
  }

#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sv + db * 16 * T::kRowBytesV + va[ks]));
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[ks][qb], o[db][qb], 0, 0, 0);
    }
  // same read-ahead for the V^T operands
  __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
  for (int j = 0; j < KS * DB - 4; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 1);
  }
  __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 1);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void chunk_attn_kernel(AttnParams p) {
  using T = Tile<D>;
  constexpr int KK = D / 32;
  constexpr int DB = D / 16;
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
  const int h = lane / 16, c16 = lane % 16;
  int ka[KK], va[KS];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ka[kk] = c16 * T::kRowBytesK + 16 * ((4 * kk + h) ^ swz<T::kChunksK>(c16));
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) va[ks] = c16 * T::kRowBytesV + 16 * ((4 * ks + h) ^ swz<8>(c16));

  LaneSlots<D> slots;
#pragma unroll
  for (int i = 0; i < T::kSlotsK; ++i)
    slots.k_off[i] =
        (unsigned)(key_of_lds_row(k_piece_row<D>(wave, lane, i)) * D + 8 * k_piece_chunk<D>(wave, lane, i)) * 2u;
  const Runs runs = load_runs(p, head);
  RunCursor cursor;
  cursor_seek<D>(runs, cursor, slots, wave, lane, key_begin);

  // Q^T B operand: lane holds head dims 32kk + 8h .. +8 of query 16qb + c16.
  bf16x8 qf[KK][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q_row = qt * QT + wave * 32 + 16 * qb + c16;
    const bool ok = q_row < p.n_queries;
    const uint16_t* qp = p.q + ((long long)(ok ? q_row : 0) * p.num_heads + head) * D + 8 * h;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk][qb] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + 32 * kk) : make_uint4(0, 0, 0, 0));
  }

  f32x4 o[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};  // running max of scaled scores (log2 domain), per query block
  float lsum[2] = {0.f, 0.f};  // this lane's share of the running sums
  float thr[2] = {-INFINITY, -INFINITY};  // raw-score level that forces a rescale

  fetch_tile<D>(runs, slots, cursor, wave, lane, t_begin * KT, key_begin, key_end, sk0, sv0);
  for (int t = t_begin; t < t_end; t += 2) {
    // buffer 0 holds tile t; tile t+1 goes to buffer 1 while t is computed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 1 < t_end) fetch_tile<D>(runs, slots, cursor, wave, lane, (t + 1) * KT, key_begin, key_end, sk1, sv1);
    attend_tile<D>(sk0, sv0, ka, va, qf, o, m, thr, lsum, p.scale_log2, t * KT + KT > key_end, t * KT, key_end, h);
    if (t + 1 >= t_end) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (t + 2 < t_end) fetch_tile<D>(runs, slots, cursor, wave, lane, (t + 2) * KT, key_begin, key_end, sk0, sv0);
    attend_tile<D>(sk1, sv1, ka, va, qf, o, m, thr, lsum, p.scale_log2, (t + 1) * KT + KT > key_end, (t + 1) * KT, key_end,
                   h);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q_row = qt * QT + wave * 32 + 16 * qb + c16;
    float ltot = lsum[qb];
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ltot), __float_as_uint(ltot), false, false);
      ltot = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(ltot), __float_as_uint(ltot), false, false);
      ltot = __uint_as_float(t[0]) + __uint_as_float(t[1]);
    }
    const float inv = 1.f / ltot;
    if (q_row >= p.n_queries) continue;
    if (p.n_splits == 1) {
      uint16_t* op = p.out + ((long long)q_row * p.num_heads + head) * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x2 lo = {(__bf16)(o[db][qb][0] * inv), (__bf16)(o[db][qb][1] * inv)};
        const bf16x2 hi = {(__bf16)(o[db][qb][2] * inv), (__bf16)(o[db][qb][3] * inv)};
        *reinterpret_cast<uint2*>(op + 16 * db) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    } else {
      const long long row = ((long long)split * p.n_queries + q_row) * p.num_heads + head;
      float* op = p.part_o + row * D + 4 * h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(op + 16 * db) =
            make_float4(o[db][qb][0] * inv, o[db][qb][1] * inv, o[db][qb][2] * inv, o[db][qb][3] * inv);
      if (h == 0) p.part_lse[row] = m[qb] + __log2f(ltot);
    }
  }
}

// Merge of the key splits: O = sum_j 2^(lse_j - M) O_j / sum_j 2^(lse_j - M).
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
  constexpr int TPR = D / 4;  // threads per (query, head) row
  const long long rows = (long long)p.n_queries * p.num_heads;
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c4 = threadIdx.x % TPR;
  // every split's log-sum-exp and values are loaded up front, so a thread has
  // all its loads in flight at once
  float lse[kAttnMaxSplits];
  float4 v[kAttnMaxSplits];
#pragma unroll
  for (int j = 0; j < kAttnMaxSplits; ++j) {
    const bool on = j < p.n_splits;
    lse[j] = on ? p.part_lse[j * rows + row] : -INFINITY;
    v[j] = on ? *reinterpret_cast<const float4*>(p.part_o + (j * rows + row) * D + 4 * c4)
              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mx = lse[0];
#pragma unroll
  for (int j = 1; j < kAttnMaxSplits; ++j) mx = fmaxf(mx, lse[j]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < kAttnMaxSplits; ++j) {
    if (j >= p.n_splits) break;
    const float w = __builtin_amdgcn_exp2f(lse[j] - mx);
    wsum += w;
    acc.x += w * v[j].x;
    acc.y += w * v[j].y;
    acc.z += w * v[j].z;
    acc.w += w * v[j].w;
  }
  const float inv = 1.f / wsum;
  const bf16x2 lo = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv)};
  const bf16x2 hi = {(__bf16)(acc.z * inv), (__bf16)(acc.w * inv)};
  *reinterpret_cast<uint2*>(p.out + row * D + 4 * c4) =
      make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

}  // namespace

hipError_t launch_chunk_attention(const AttnParams& p, int head_dim, hipStream_t s) {
  if (p.n_queries <= 0 || p.n_keys <= 0 || p.n_splits < 1) return hipErrorInvalidValue;
  const int units = p.q_tiles * p.num_heads * p.n_splits;
  const int combine_blocks = (int)(((long long)p.n_queries * p.num_heads * (head_dim / 4) + 255) / 256);
  if (head_dim == 128) {
    hipLaunchKernelGGL(chunk_attn_kernel<128>, dim3(units), dim3(kThreads), 0, s, p);
    if (p.n_splits > 1) hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(combine_blocks), dim3(256), 0, s, p);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL(chunk_attn_kernel<64>, dim3(units), dim3(kThreads), 0, s, p);
    if (p.n_splits > 1) hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(combine_blocks), dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ckv
