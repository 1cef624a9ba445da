// 3D RoPE + K/V append for one chunk, the text-context store for
// cross-attention, and the K/V copy-out used for checks.
//
// RoPE ("Learning Video Generation from the Wan2.2 Source Code", Chapter 4,
// "3D RoPE"): the head dim is split into a time band of d - 4(d/6) dims and
// height and width bands of 2(d/6) dims each; every adjacent pair
// (x[2p], x[2p+1]) is a complex number multiplied by e^{i * pos * w}, where
// pos is the token's frame, patch row or patch column for the pair's band.
// q and k are rotated, v is not.  The cos/sin values come from tables that
// rope_table_kernel builds once per cache in float64 (w_j = theta^(-2j/D_band)
// per band, the band's own width, then cos and sin of pos * w_j) and rounds
// once to float32; the rotation itself is float32 with one bf16 rounding
// (nearest-even) at the end.
//
// QK-Norm ("Learning Video Generation from the Wan2.2 Source Code", Chapter 4,
// "3D RoPE" detail paragraph: q and k each pass an RMSNorm after their linear
// layers), when asked for: the wave that rotates a token's q (or its k) holds
// all of its H*d values, so it takes their mean of squares (float32, a wave
// reduction), scales each value by 1/sqrt(mean + eps) and its channel's gain,
// rounds to bf16 (the norm's output precision) and rotates that -- the norm
// costs no extra pass over q and k.
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

// Streaming 16-byte store: the outputs are not read again by this kernel, and
// marking them nontemporal keeps them from displacing the inputs in the
// caches (measured: 11.5 -> 10.2 us per 880-token append).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ inline void store_nt(const uint4& v, uint16_t* p) {
  const u32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(p));
}

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

// x (8 bf16) * inv * gain[0..7], rounded to bf16 once.
__device__ inline uint4 norm8(const uint4& in, float inv, const float* __restrict__ gain) {
  const float4 g0 = *reinterpret_cast<const float4*>(gain);
  const float4 g1 = *reinterpret_cast<const float4*>(gain + 4);
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const uint32_t w_in[4] = {in.x, in.y, in.z, in.w};
  uint32_t w_out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float y0 = bf16_to_f32((uint16_t)(w_in[j] & 0xFFFFu)) * inv * g[2 * j];
    const float y1 = bf16_to_f32((uint16_t)(w_in[j] >> 16)) * inv * g[2 * j + 1];
    w_out[j] = (uint32_t)f32_to_bf16(y0) | ((uint32_t)f32_to_bf16(y1) << 16);
  }
  return make_uint4(w_out[0], w_out[1], w_out[2], w_out[3]);
}

// Wave sum of a float over its 64 lanes.
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline float sum_sq8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16_to_f32((uint16_t)(w[j] & 0xFFFFu)), b = bf16_to_f32((uint16_t)(w[j] >> 16));
    s += a * a + b * b;
  }
  return s;
}

constexpr int kGroup = 8;  // 16-byte chunks a lane holds at once (512 per wave)

// Two kinds of workgroup in one launch (qk_blocks of the first kind, one per
// 64 tokens and head of the second).
//  * q/k workgroups rotate q and k.  Without the QK-Norm: one thread per
//    16-byte chunk (flat over token x chunk).  With it: one wave per token
//    and tensor, covering q (or k) of all heads (the token's whole projected
//    vector, H*d values): consecutive lanes take consecutive 16-byte chunks,
//    so loads and stores are fully coalesced, and the wave holds every value
//    for the mean of squares (a wave reduction) before it scales, rounds and
//    rotates.
//  * V workgroups: V^T for 64 tokens of one head, transposed through LDS.
// The longer kind is dispatched first, so that it does not form the tail:
// without the norm the V workgroups (load, barrier, transposed stores) come
// first (measured: 10.1 -> 9.2 us per 880-token append), with it the q/k
// waves, which each cover a token's whole vector.
template <int D, bool kNorm>
__global__ __launch_bounds__(kThreads) void rope_append_kernel(RopeAppendParams p, int qk_blocks) {
  constexpr int C8 = D / 8;                   // 16-byte chunks per head row
  constexpr int Pt = (D - 4 * (D / 6)) / 2;
  constexpr int Ph = (2 * (D / 6)) / 2;
  __shared__ uint16_t sv[kTok][D + 8];        // V tile, padded rows
  const int H = p.num_heads;
  const float2* tab_t = reinterpret_cast<const float2*>(p.cos_sin);
  const float2* tab_h = tab_t + p.n_frames_table * Pt;
  const float2* tab_w = tab_h + p.grid_h * Ph;
  const int tok_blocks = (p.n_tokens + kTok - 1) / kTok;
  const int v_blocks = tok_blocks * H;
  // index among the q/k workgroups (qb) or among the V workgroups (vb);
  // the other one is negative
  const int qb = kNorm ? (int)blockIdx.x : (int)blockIdx.x - v_blocks;
  const int vb = kNorm ? (int)blockIdx.x - qk_blocks : (int)blockIdx.x;

  if (!kNorm && qb >= 0) {
    // Without the norm the rotation is elementwise: one thread per 16-byte
    // chunk of q and of k (a flat grid over token x chunk, like a copy), the
    // two loads issued before any table lookup.
    const int W8 = H * C8;  // chunks per token
    const long long e = (long long)qb * kThreads + threadIdx.x;
    if (e >= (long long)p.n_tokens * W8) return;
    const int tok = (int)(e / W8);
    const int c = (int)(e - (long long)tok * W8);
    const uint4 qv = *reinterpret_cast<const uint4*>(p.q + e * 8);
    const uint4 kv = *reinterpret_cast<const uint4*>(p.k + e * 8);
    const int per_frame = p.grid_h * p.grid_w;
    const int fl = tok / per_frame;
    const int rem = tok - fl * per_frame;
    const int row = rem / p.grid_w;
    const int col = rem - row * p.grid_w;
    const int head = c / C8, cc = c % C8;
    uint4 qo, ko;
    rotate8<D>(qv, qo, cc * 4, p.first_frame + fl, row, col, tab_t, tab_h, tab_w);
    rotate8<D>(kv, ko, cc * 4, p.first_frame + fl, row, col, tab_t, tab_h, tab_w);
    store_nt(qo, p.q_rot + e * 8);
    store_nt(ko, p.k_dst + head * p.k_head_stride + (long long)tok * D + cc * 8);
    return;
  }
  if (kNorm && vb < 0) {
    // one wave per (token, tensor): q and k of a token are normalised on
    // their own, so two waves share the token
    const int g = qb * (kThreads / 64) + threadIdx.x / 64;
    const int tok = g >> 1;
    const bool is_k = (g & 1) != 0;
    const int lane = threadIdx.x % 64;
    if (tok >= p.n_tokens) return;  // no barrier on this path
    const int per_frame = p.grid_h * p.grid_w;
    const int fl = tok / per_frame;
    const int rem = tok - fl * per_frame;
    const int row = rem / p.grid_w;
    const int col = rem - row * p.grid_w;
    const int frame = p.first_frame + fl;
    const int W8 = H * C8;                    // chunks per token
    const long long base = (long long)tok * H * D;
    const uint16_t* src = is_k ? p.k : p.q;
    const float* gain = is_k ? p.k_gain : p.q_gain;
    float inv = 1.f;
    if (W8 > 64 * kGroup) {                   // wide tokens: a first pass for the norm
      float sq = 0.f;
      for (int c = lane; c < W8; c += 64) sq += sum_sq8(*reinterpret_cast<const uint4*>(src + base + c * 8));
      inv = 1.f / sqrtf(wave_sum(sq) / (H * D) + p.eps);
    }
    for (int g0 = 0; g0 < W8; g0 += 64 * kGroup) {
      uint4 xv[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int c = g0 + lane + 64 * i;
        if (c < W8) xv[i] = *reinterpret_cast<const uint4*>(src + base + c * 8);
      }
      if (W8 <= 64 * kGroup) {
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
          if (g0 + lane + 64 * i < W8) sq += sum_sq8(xv[i]);
        inv = 1.f / sqrtf(wave_sum(sq) / (H * D) + p.eps);
      }
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int c = g0 + lane + 64 * i;
        if (c < W8) {
          const int head = c / C8, cc = c % C8;
          uint4 xo;
          rotate8<D>(norm8(xv[i], inv, gain + c * 8), xo, cc * 4, frame, row, col, tab_t, tab_h, tab_w);
          // channel c*8.. = head*d + 8*cc..
          store_nt(xo, is_k ? p.k_dst + head * p.k_head_stride + (long long)tok * D + cc * 8 : p.q_rot + base + c * 8);
        }
      }
    }
    return;
  }

  const int head = vb / tok_blocks;
  const int tok0 = (vb % tok_blocks) * kTok;
#pragma unroll
  for (int it = 0; it < (kTok * C8) / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int t = idx / C8;
    const int c = idx % C8;
    const int tok = tok0 + t;
    if (tok < p.n_tokens)
      *reinterpret_cast<uint4*>(&sv[t][c * 8]) =
          *reinterpret_cast<const uint4*>(p.v + ((long long)tok * H + head) * D + c * 8);
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
      store_nt(make_uint4(w[0], w[1], w[2], w[3]),
               p.vt_dst + head * p.vt_head_stride + (long long)dim * p.vt_row_stride + tok0 + t);
    }
  }
}

// The text context of one layer into the attention store.  Blocks
// [0, k_blocks) copy K rows ([n][H][d] -> [H][max][d], 16 bytes a lane);
// the rest write V^T for 64 context rows of one head through LDS, zero past
// n_text so that every V^T column the attention reads is finite.
template <int D>
__global__ __launch_bounds__(kThreads) void text_store_kernel(TextStoreParams p, int k_blocks) {
  constexpr int C8 = D / 8;
  __shared__ uint16_t sv[kTok][D + 8];
  const int H = p.num_heads;
  if ((int)blockIdx.x < k_blocks) {
    const long long e = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (e >= (long long)p.n_text * H * C8) return;
    const int c = (int)(e % C8);
    const long long th = e / C8;
    const int head = (int)(th % H);
    const int tok = (int)(th / H);
    *reinterpret_cast<uint4*>(p.k_dst + ((long long)head * p.max_text + tok) * D + c * 8) =
        *reinterpret_cast<const uint4*>(p.k + e * 8);
    return;
  }
  const int vb = blockIdx.x - k_blocks;
  const int head = vb / (p.max_text / kTok);
  const int tok0 = (vb % (p.max_text / kTok)) * kTok;
#pragma unroll
  for (int it = 0; it < (kTok * C8) / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int t = idx / C8;
    const int c = idx % C8;
    const int tok = tok0 + t;
    *reinterpret_cast<uint4*>(&sv[t][c * 8]) =
        tok < p.n_text ? *reinterpret_cast<const uint4*>(p.v + ((long long)tok * H + head) * D + c * 8)
                       : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < (kTok / 8 * D) / kThreads; ++it) {
    const int idx = threadIdx.x + it * kThreads;
    const int g = idx % (kTok / 8);
    const int dim = idx / (kTok / 8);
    const int t = g * 8;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (uint32_t)sv[t + 2 * j][dim] | ((uint32_t)sv[t + 2 * j + 1][dim] << 16);
    *reinterpret_cast<uint4*>(p.vt_dst + ((long long)head * D + dim) * p.max_text + tok0 + t) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// The angle tables: (cos, sin) float2 for [frames][Pt] | [grid_h][Ph] |
// [grid_w][Pw] pairs, evaluated in float64 and rounded once to float32.
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableParams p) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int nt = p.frames * (p.band_t / 2), nh = p.grid_h * (p.band_h / 2), nw = p.grid_w * (p.band_w / 2);
  if (i >= nt + nh + nw) return;
  int pos, j, width;
  if (i < nt) {
    pos = i / (p.band_t / 2), j = i % (p.band_t / 2), width = p.band_t;
  } else if (i < nt + nh) {
    pos = (i - nt) / (p.band_h / 2), j = (i - nt) % (p.band_h / 2), width = p.band_h;
  } else {
    pos = (i - nt - nh) / (p.band_w / 2), j = (i - nt - nh) % (p.band_w / 2), width = p.band_w;
  }
  const double a = (double)pos * pow(p.theta, -2.0 * j / (double)width);
  p.out[i] = make_float2((float)cos(a), (float)sin(a));
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
  if (p.n_tokens <= 0 || p.num_heads <= 0) return hipErrorInvalidValue;
  const bool norm = p.q_gain != nullptr;
  // the norm needs a token's whole q (or k) vector in one wave: two waves per
  // token; the plain rotation is a flat grid over 16-byte chunks
  const long long chunks = (long long)p.n_tokens * p.num_heads * (head_dim / 8);
  const int qk_blocks = norm ? (2 * p.n_tokens + kThreads / 64 - 1) / (kThreads / 64) : (int)((chunks + kThreads - 1) / kThreads);
  const int v_blocks = ((p.n_tokens + kTok - 1) / kTok) * p.num_heads;
  const dim3 grid(qk_blocks + v_blocks);
  if (head_dim == 128 && norm)
    hipLaunchKernelGGL((rope_append_kernel<128, true>), grid, dim3(kThreads), 0, s, p, qk_blocks);
  else if (head_dim == 128)
    hipLaunchKernelGGL((rope_append_kernel<128, false>), grid, dim3(kThreads), 0, s, p, qk_blocks);
  else if (head_dim == 64 && norm)
    hipLaunchKernelGGL((rope_append_kernel<64, true>), grid, dim3(kThreads), 0, s, p, qk_blocks);
  else if (head_dim == 64)
    hipLaunchKernelGGL((rope_append_kernel<64, false>), grid, dim3(kThreads), 0, s, p, qk_blocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_text_store(const TextStoreParams& p, int head_dim, hipStream_t s) {
  if (p.n_text <= 0 || p.n_text > p.max_text || p.max_text % kTok != 0 || p.num_heads <= 0) return hipErrorInvalidValue;
  const long long chunks = (long long)p.n_text * p.num_heads * (head_dim / 8);
  const int k_blocks = (int)((chunks + kThreads - 1) / kThreads);
  const dim3 grid(k_blocks + p.num_heads * (p.max_text / kTok));
  if (head_dim == 128)
    hipLaunchKernelGGL(text_store_kernel<128>, grid, dim3(kThreads), 0, s, p, k_blocks);
  else if (head_dim == 64)
    hipLaunchKernelGGL(text_store_kernel<64>, grid, dim3(kThreads), 0, s, p, k_blocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rope_table(const RopeTableParams& p, hipStream_t s) {
  const int n = p.frames * (p.band_t / 2) + p.grid_h * (p.band_h / 2) + p.grid_w * (p.band_w / 2);
  if (n <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_table_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p);
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
