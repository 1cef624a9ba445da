// Same-step chunk attention on CDNA4 (gfx950): a flash-style kernel with
// bf16 MFMA for both products and an fp32 online softmax.
//
// What it computes ("PhysisServe -- Wan2.2 5B" model card, "Inference
// profile"): for every head and query, softmax(scale * q K_win^T) V_win over
// the window [sink | same-step ring window | own chunk], no mask.  The
// window is not concatenated: it arrives as up to three runs of keys (the
// sink, then up to two runs of ring slots) and every 8-key group of a tile is
// addressed in the run that holds it.
//
// Tiling.  A workgroup is 4 waves; each wave owns 32 query rows of one head
// (128 rows per workgroup).  Keys stream through LDS in tiles of 64: K rows
// [64][d] and V^T [d][64], padded so that the 16-byte MFMA operand reads are
// bank-conflict free.  Per tile and wave:
//   S^T[64 keys x 32 queries] = K_tile Q^T   (v_mfma_f32_32x32x16_bf16)
// with the queries as the MFMA's N columns, so one lane holds 32 scores of a
// single query and the row max / row sum need only one cross-half exchange
// (v_permlane32_swap).  The K rows feeding the A operand are permuted
// (bits 2 and 3 of the row swapped) so that the 8 scores a lane holds for
// each 16-key step of the next product are 8 consecutive keys:
//   O^T[d x 32 queries] += V^T_tile P^T       (v_mfma_f32_32x32x16_bf16)
// takes P straight from registers (converted to bf16) and V^T from LDS with
// one 16-byte read per lane.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int QT = kAttnQueryTile;  // 128
constexpr int KT = kAttnKeyTile;    // 64
constexpr int kThreads = 256;
constexpr int kXcds = 8;

template <int D>
struct Smem {
  uint16_t k[KT][D + 8];   // key rows, padded by 16 bytes
  uint16_t vt[D][KT + 8];  // head-dim rows of V^T, padded by 16 bytes
};

__device__ inline bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Run holding key j (runs are ordered and end at seg_end[0..2]).
__device__ inline int run_of(const AttnParams& p, int j) { return (j >= p.seg_end[0]) + (j >= p.seg_end[1]); }

template <int D>
__device__ inline const uint16_t* key_row(const AttnParams& p, int head, int j) {
  const int r = run_of(p, j);
  const int start = r == 0 ? 0 : (r == 1 ? p.seg_end[0] : p.seg_end[1]);
  const uint16_t* base = r == 0 ? p.k[0] : (r == 1 ? p.k[1] : p.k[2]);
  const long long hs = r == 0 ? p.k_head_stride[0] : (r == 1 ? p.k_head_stride[1] : p.k_head_stride[2]);
  return base + head * hs + (long long)(j - start) * D;
}

__device__ inline const uint16_t* vt_col(const AttnParams& p, int head, int dim, int j) {
  const int r = run_of(p, j);
  const int start = r == 0 ? 0 : (r == 1 ? p.seg_end[0] : p.seg_end[1]);
  const uint16_t* base = r == 0 ? p.vt[0] : (r == 1 ? p.vt[1] : p.vt[2]);
  const long long hs = r == 0 ? p.vt_head_stride[0] : (r == 1 ? p.vt_head_stride[1] : p.vt_head_stride[2]);
  const int rs = r == 0 ? p.vt_row_stride[0] : (r == 1 ? p.vt_row_stride[1] : p.vt_row_stride[2]);
  return base + head * hs + (long long)dim * rs + (j - start);
}

template <int D>
struct TileRegs {
  static constexpr int kK = KT * (D / 8) / kThreads;  // 16-byte K chunks per thread
  static constexpr int kV = D * (KT / 8) / kThreads;  // 16-byte V^T chunks per thread
  uint4 k[kK];
  uint4 v[kV];
};

template <int D>
__device__ inline void load_tile(const AttnParams& p, int head, int t0, int key_end, TileRegs<D>& r) {
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kK; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    const int row = idx / (D / 8), c = idx % (D / 8);
    const int j = t0 + row;
    r.k[i] = j < key_end ? *reinterpret_cast<const uint4*>(key_row<D>(p, head, j) + c * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kV; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    const int dim = idx / (KT / 8), g = idx % (KT / 8);
    const int j = t0 + 8 * g;  // runs are multiples of 8 keys: a group never straddles two runs
    r.v[i] = j < key_end ? *reinterpret_cast<const uint4*>(vt_col(p, head, dim, j)) : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ inline void store_tile(Smem<D>& sm, const TileRegs<D>& r) {
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kK; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    *reinterpret_cast<uint4*>(&sm.k[idx / (D / 8)][(idx % (D / 8)) * 8]) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kV; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    *reinterpret_cast<uint4*>(&sm.vt[idx / (KT / 8)][(idx % (KT / 8)) * 8]) = r.v[i];
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void chunk_attn_kernel(AttnParams p) {
  constexpr int KK = D / 16;  // 16-deep steps of the QK^T product
  constexpr int MO = D / 32;  // 32-row head-dim blocks of O^T
  __shared__ Smem<D> sm;

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

  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int half = lane / 32, col = lane % 32;
  const int q_row = qt * QT + wave * 32 + col;
  const bool q_valid = q_row < p.n_queries;
  // A-operand row -> key row of the tile: swap bits 2 and 3.
  const int prow = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);

  bf16x8 qf[KK];
  {
    const uint16_t* qp = p.q + ((long long)(q_valid ? q_row : 0) * p.num_heads + head) * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = as_bf16x8(q_valid ? *reinterpret_cast<const uint4*>(qp + 16 * kk) : make_uint4(0, 0, 0, 0));
  }

  f32x16 o[MO];
#pragma unroll
  for (int mo = 0; mo < MO; ++mo)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mo][i] = 0.f;
  float m = -INFINITY;  // running max of scaled scores (log2 domain), same in both halves
  float lsum = 0.f;     // this lane's share of the running sum

  TileRegs<D> regs;
  load_tile<D>(p, head, t_begin * KT, key_end, regs);
  store_tile<D>(sm, regs);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int t0 = t * KT;
    if (t + 1 < t_end) load_tile<D>(p, head, t0 + KT, key_end, regs);

    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[mb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.k[32 * mb + prow][16 * kk + 8 * half]));
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[mb], 0, 0, 0);
      }

    // Lane value (mb, i) is the score of tile key 32mb + 16(i/8) + 8*half + i%8.
    float mloc = -INFINITY;
    const bool tail = t0 + KT > key_end;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mb][i] * p.scale_log2;
        if (tail && t0 + 32 * mb + 16 * (i / 8) + 8 * half + (i % 8) >= key_end) x = -INFINITY;
        s[mb][i] = x;
        mloc = fmaxf(mloc, x);
      }
    const float m_new = fmaxf(m, pair_max(mloc));
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float psum = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[mb][i] - m_new);
        psum += e;
        pf[2 * mb + i / 8][i % 8] = (__bf16)e;
      }
    lsum = lsum * alpha + psum;
    m = m_new;
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mo][i] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mo = 0; mo < MO; ++mo) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(&sm.vt[32 * mo + col][16 * kb + 8 * half]));
        o[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kb], o[mo], 0, 0, 0);
      }

    __syncthreads();
    if (t + 1 < t_end) store_tile<D>(sm, regs);
    __syncthreads();
  }

  const float ltot = pair_sum(lsum);
  const float inv = 1.f / ltot;
  if (!q_valid) return;
  // O^T value (mo, i) is head-dim 32mo + 8(i/4) + 4*half + i%4 of query q_row.
  if (p.n_splits == 1) {
    uint16_t* op = p.out + ((long long)q_row * p.num_heads + head) * D + 4 * half;
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t w[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const __bf16 lo = (__bf16)(o[mo][4 * g + 2 * j] * inv);
          const __bf16 hi = (__bf16)(o[mo][4 * g + 2 * j + 1] * inv);
          w[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *reinterpret_cast<uint2*>(op + 32 * mo + 8 * g) = make_uint2(w[0], w[1]);
      }
  } else {
    const long long row = ((long long)split * p.n_queries + q_row) * p.num_heads + head;
    float* op = p.part_o + row * D + 4 * half;
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(op + 32 * mo + 8 * g) =
            make_float4(o[mo][4 * g] * inv, o[mo][4 * g + 1] * inv, o[mo][4 * g + 2] * inv, o[mo][4 * g + 3] * inv);
    if (half == 0) p.part_lse[row] = m + __log2f(ltot);
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
  float mx = -INFINITY;
  for (int j = 0; j < p.n_splits; ++j) mx = fmaxf(mx, p.part_lse[j * rows + row]);
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < p.n_splits; ++j) {
    const float w = __builtin_amdgcn_exp2f(p.part_lse[j * rows + row] - mx);
    const float4 v = *reinterpret_cast<const float4*>(p.part_o + (j * rows + row) * D + 4 * c4);
    wsum += w;
    acc.x += w * v.x;
    acc.y += w * v.y;
    acc.z += w * v.z;
    acc.w += w * v.w;
  }
  const float inv = 1.f / wsum;
  const __bf16 b0 = (__bf16)(acc.x * inv), b1 = (__bf16)(acc.y * inv), b2 = (__bf16)(acc.z * inv),
               b3 = (__bf16)(acc.w * inv);
  const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
  const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
  *reinterpret_cast<uint2*>(p.out + row * D + 4 * c4) = make_uint2(w0, w1);
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
