// 3D RoPE + K/V append for one chunk, and the K/V copy-out used for checks.
//
// RoPE ("Learning Video Generation from the Wan2.2 Source Code", Chapter 4,
// "3D RoPE"): the head dim is split into a time band of d - 4(d/6) dims and
// height and width bands of 2(d/6) dims each; every adjacent pair
// (x[2p], x[2p+1]) is a complex number multiplied by e^{i * pos * w}, where
// pos is the token's frame, patch row or patch column for the pair's band.
// q and k are rotated, v is not.  The cos/sin values come from tables built
// on the host in float64 and rounded once to float32; the rotation itself is
// float32 with one bf16 rounding (nearest-even) at the end.
//
// Store layout written here (read by the attention kernel):
//   K rows  [H][rows][d]   -- one contiguous d-vector per key;
//   V^T     [H][d][cols]   -- keys contiguous along a head-dim row, so the
//                             PV product can take 8 consecutive keys of one
//                             head-dim row with a single 16-byte load.
// The transpose goes through LDS.  The kernel is a streaming copy with a
// rotation: 3 reads and 3 writes of [n][H][d] bf16, HBM-bound.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ckv {
namespace {

constexpr int kTok = 64;        // tokens per workgroup (one head)
constexpr int kThreads = 256;

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bf16, round to nearest even (inputs are finite).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D>
__device__ inline void rotate8(const uint4& in, uint4& out, int pair0, int frame, int row, int col,
                               const float2* __restrict__ tab_t, const float2* __restrict__ tab_h,
                               const float2* __restrict__ tab_w) {
  constexpr int Pt = (D - 4 * (D / 6)) / 2;  // pairs in the time band
  constexpr int Ph = (2 * (D / 6)) / 2;      // pairs in the height band
  constexpr int Pw = Ph;                     // pairs in the width band
  const uint32_t w_in[4] = {in.x, in.y, in.z, in.w};
  uint32_t w_out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = pair0 + j;
    float2 cs;
    if (p < Pt)
      cs = tab_t[frame * Pt + p];
    else if (p < Pt + Ph)
      cs = tab_h[row * Ph + (p - Pt)];
    else
      cs = tab_w[col * Pw + (p - Pt - Ph)];
    const float x0 = bf16_to_f32((uint16_t)(w_in[j] & 0xFFFFu));
    const float x1 = bf16_to_f32((uint16_t)(w_in[j] >> 16));
    const float y0 = x0 * cs.x - x1 * cs.y;
    const float y1 = x0 * cs.y + x1 * cs.x;
    w_out[j] = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
  }
  out = make_uint4(w_out[0], w_out[1], w_out[2], w_out[3]);
}

template <int D>
__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeAppendParams p) {
  constexpr int C8 = D / 8;                   // 16-byte chunks per head row
  constexpr int Pt = (D - 4 * (D / 6)) / 2;
  constexpr int Ph = (2 * (D / 6)) / 2;
  __shared__ uint16_t sv[kTok][D + 8];        // V tile, padded rows

  const int head = blockIdx.y;
  const int tok0 = blockIdx.x * kTok;
  const int H = p.num_heads;
  const int per_frame = p.grid_h * p.grid_w;
  const float2* tab_t = reinterpret_cast<const float2*>(p.cos_sin);
  const float2* tab_h = tab_t + p.n_frames_table * Pt;
  const float2* tab_w = tab_h + p.grid_h * Ph;

  // q and k: rotate 8 elements (4 pairs) per 16-byte chunk; v: stage in LDS.
#pragma unroll
  for (int it = 0; it < (kTok * C8) / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int t = idx / C8;
    const int c = idx % C8;
    const int tok = tok0 + t;
    if (tok < p.n_tokens) {
      const int fl = tok / per_frame;
      const int rem = tok - fl * per_frame;
      const int row = rem / p.grid_w;
      const int col = rem - row * p.grid_w;
      const int frame = p.first_frame + fl;
      const long long src = ((long long)tok * H + head) * D + c * 8;
      const uint4 qv = *reinterpret_cast<const uint4*>(p.q + src);
      const uint4 kv = *reinterpret_cast<const uint4*>(p.k + src);
      const uint4 vv = *reinterpret_cast<const uint4*>(p.v + src);
      uint4 qo, ko;
      rotate8<D>(qv, qo, c * 4, frame, row, col, tab_t, tab_h, tab_w);
      rotate8<D>(kv, ko, c * 4, frame, row, col, tab_t, tab_h, tab_w);
      *reinterpret_cast<uint4*>(p.q_rot + src) = qo;
      *reinterpret_cast<uint4*>(p.k_dst + head * p.k_head_stride + (long long)tok * D + c * 8) = ko;
      *reinterpret_cast<uint4*>(&sv[t][c * 8]) = vv;
    }
  }
  __syncthreads();
  // V^T: each thread writes 8 consecutive tokens of one head-dim row.
#pragma unroll
  for (int it = 0; it < (kTok / 8 * D) / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int g = idx % (kTok / 8);  // token group
    const int dim = idx / (kTok / 8);
    const int t = g * 8;
    if (tok0 + t < p.n_tokens) {  // n_tokens is a multiple of 8
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = (uint32_t)sv[t + 2 * j][dim] | ((uint32_t)sv[t + 2 * j + 1][dim] << 16);
      *reinterpret_cast<uint4*>(p.vt_dst + head * p.vt_head_stride + (long long)dim * p.vt_row_stride + tok0 + t) =
          make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void copy_kv_kernel(CopyKVParams p) {
  const long long total = (long long)p.n_tokens * p.num_heads * D;
  for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    const int dim = (int)(e % D);
    const long long th = e / D;
    const int head = (int)(th % p.num_heads);
    const int tok = (int)(th / p.num_heads);
    p.k_out[e] = p.k_src[head * p.k_head_stride + (long long)tok * D + dim];
    p.v_out[e] = p.vt_src[head * p.vt_head_stride + (long long)dim * p.vt_row_stride + tok];
  }
}

}  // namespace

hipError_t launch_rope_append(const RopeAppendParams& p, int head_dim, hipStream_t s) {
  dim3 grid((p.n_tokens + kTok - 1) / kTok, p.num_heads);
  if (head_dim == 128)
    hipLaunchKernelGGL(rope_append_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(rope_append_kernel<64>, grid, dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_copy_kv(const CopyKVParams& p, int head_dim, hipStream_t s) {
  const long long total = (long long)p.n_tokens * p.num_heads * head_dim;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (head_dim == 128)
    hipLaunchKernelGGL(copy_kv_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL(copy_kv_kernel<64>, dim3(blocks), dim3(256), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ckv
