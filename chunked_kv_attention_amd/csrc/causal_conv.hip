// Streaming causal 3D convolution on CDNA4 (gfx950): implicit GEMM on bf16
// MFMA with a 2-frame temporal cache.
//
// What it computes ("Learning Video Generation from the Wan2.2 Source Code",
// Chapter 2, "Causal Convolution and Streaming Inference"): Conv3d with all
// time padding in front (kt - 1 frames), symmetric spatial padding, fed one
// chunk of frames at a time; the frames before the chunk come from a cache
// of the last two input frames of the stream (zeros before the video).
//
// GEMM view.  Output y^T[c_out][pixel] = sum over (tap, c_in) of
// W[tap][c_out][c_in] * X_tap[pixel][c_in], where X_tap is the input shifted
// by the tap.  The K dimension runs tap-major over blocks of 64 input
// channels; no im2col buffer exists: each block of X is gathered straight
// from the chunk, the cache or a zero row.
//
// Tiling.  A workgroup is 4 waves and owns 128 output channels x 128 output
// pixels (pixels in [frame][row][col] order, so a tile may span rows and
// frames); wave w owns channel half w & 1 and pixel half w >> 1, i.e. a
// 64 x 64 block of 4 x 4 MFMA outputs.  Per 64-channel block, a 16 KB W tile
// ([128 c_out][64 c_in]) and a 16 KB X tile ([128 pixels][64 c_in]) land in
// LDS by global_load_lds_dwordx4, 16-byte chunks of each 128-byte row
// XOR-swizzled so that the operand reads (16 lanes on 16 consecutive rows,
// one logical chunk) are conflict-free.  Two buffers alternate with one
// barrier per block; block j+1 is in flight while block j is computed.
//
// Gather.  Each lane fetches fixed rows of the X tile; when the tap changes
// it recomputes, for each of its rows, the source pixel (frame t + a - (kt-1),
// row + b - (kh-1)/2, column + c - (kw-1)/2): a frame of the chunk, a cache
// slot (global frame index mod 2) or, outside the video, the zero row.
//
// Products use v_mfma_f32_16x16x32_bf16 with the weights as the A operand
// (rows = output channels) and the pixels as the B columns, so a lane ends
// with 4 consecutive output channels of one pixel: one 8-byte store each.
//
// Occupancy.  A one-frame chunk of a small grid has too few tiles for 256
// CUs, and a larger call may leave a last, partly filled round of tiles;
// such tiles are split by time offset (kt parts, one input frame each),
// every part writes float32 partials, and a second kernel adds them and the
// bias and rounds once.
#include <hip/hip_runtime.h>

#include "kernels.hpp"

namespace ckv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kPix = kConvPixelTile;      // 128 output pixels per workgroup
constexpr int kCout = kConvChannelTile;   // 128 output channels per workgroup
constexpr int kCb = 64;                   // input channels per LDS block
constexpr int kRowBytes = 2 * kCb;        // 128: 8 chunks of 16 bytes
constexpr int kTileBytes = 128 * kRowBytes;
constexpr int kSlots = kTileBytes / 1024 / kWaves;  // fetches per wave per tile
constexpr int kXcds = 8;
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
static_assert(kPix == 128 && kCout == 128, "tile rows are 128 on both operands");

// chunk swizzle of 128-byte LDS row r: two rows fill the 64 banks once, so
// rows 2m and 2m+1 differ in bank half and rows with different m in chunk
__device__ inline int swz(int r) { return (r >> 1) & 7; }

__device__ inline bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

__device__ inline const char* uni(const void* ptr) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(ptr);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

template <class T>
__device__ inline void opaque(T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
}

// One 16-byte-per-lane global -> LDS transfer (lane l lands at lds + 16 l).
__device__ inline void lds_dma16(const void* src, lds_void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

// The rows a lane fetches: slot i of wave w is LDS block w + 4 i (1 KB = 8
// rows), lane l lands in row 8 (w + 4 i) + l / 8 at physical chunk l % 8,
// which holds logical chunk (l % 8) ^ swz(row).
__device__ inline int slot_row(int w, int l, int i) { return 8 * (w + kWaves * i) + l / 8; }
__device__ inline int slot_chunk(int w, int l, int i) { return (l % 8) ^ swz(slot_row(w, l, i)); }

// Source of one X-tile row for one tap: the row's pixel shifted by the tap.
struct PixelOfRow {
  int t, y, x;  // frame within the chunk, grid row, grid column
  bool in;      // the row is a real output pixel
};

__device__ inline const char* gather_row(const ConvParams& p, const PixelOfRow& px, int chunk, int dt, int dy,
                                         int dx) {
  const int tl = px.t + dt;  // frame relative to the chunk's first (>= -2)
  const int yy = px.y + dy, xx = px.x + dx;
  const long long frame_bytes = (long long)p.height * p.width * p.c_in * 2;
  const long long pix_bytes = ((long long)yy * p.width + xx) * p.c_in * 2;
  bool ok = px.in && yy >= 0 && yy < p.height && xx >= 0 && xx < p.width;
  const char* base;
  if (tl >= 0) {
    base = reinterpret_cast<const char*>(p.x) + tl * frame_bytes;
  } else {
    const long long g = p.k0 + tl;  // global frame index; < 0 is before the video
    ok = ok && g >= 0;
    base = reinterpret_cast<const char*>(p.cache) + (g & 1) * frame_bytes;
  }
  return ok ? base + pix_bytes + 16 * chunk : reinterpret_cast<const char*>(p.zero) + 16 * chunk;
}

__global__ __launch_bounds__(kThreads, 2) void causal_conv_kernel(ConvParams p) {
  __shared__ __attribute__((aligned(1024))) char sw0[kTileBytes], sw1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char sx0[kTileBytes], sx1[kTileBytes];

  // Work item -> (unit, part).  Blocks [0, whole) run whole units, the rest
  // run the parts of the later units, part fastest.  Within each of the two
  // ranges every XCD gets a contiguous run of items, so the tiles that share
  // X share its L2 (blocks go round-robin over the 8 XCDs).
  const int n_ct = p.c_out / kCout;
  const int units = p.m_tiles * n_ct;
  const bool in_whole = (int)blockIdx.x < p.whole;
  const int r0 = in_whole ? 0 : p.whole;
  const int rlen = in_whole ? p.whole : (units - p.whole) * p.splits;
  const int b = blockIdx.x - r0;
  const int xcd = b % kXcds, li = b / kXcds;
  const int per = rlen / kXcds, extra = rlen % kXcds;
  const int item = xcd * per + (xcd < extra ? xcd : extra) + li;
  const int parts = in_whole ? 1 : p.splits;
  const int split = in_whole ? 0 : item % p.splits;
  const int unit = in_whole ? item : p.whole + item / p.splits;
  const int mt = unit / n_ct, ct = unit % n_ct;
  const int m0 = mt * kPix, cout0 = ct * kCout;
  const int n_pix = p.frames * p.height * p.width;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64), lane = threadIdx.x % 64;
  const int h = lane / 16, c16 = lane % 16;
  const int half_c = wave & 1, half_p = wave >> 1;

  // this lane's fetch rows: W offsets within a (tap, channel block) slab and
  // the pixel behind each X row
  unsigned w_off[kSlots];
  PixelOfRow px[kSlots];
  int xchunk[kSlots];
  const int hw = p.height * p.width;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    const int r = slot_row(wave, lane, i);
    xchunk[i] = slot_chunk(wave, lane, i);
    w_off[i] = (unsigned)(((cout0 + r) * p.c_in + 8 * xchunk[i]) * 2);
    const int m = m0 + r;
    px[i].in = m < n_pix;
    const int mm = px[i].in ? m : 0;
    px[i].t = mm / hw;
    const int rem = mm % hw;
    px[i].y = rem / p.width;
    px[i].x = rem % p.width;
  }

  // operand read offsets within a tile (row 16 blk + c16, chunk 4 s + h)
  int rd[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) rd[s] = c16 * kRowBytes + 16 * ((4 * s + h) ^ swz(c16));

  const int n_cb = p.c_in / kCb;
  // this workgroup's K range: all taps, or the taps of time offset `split`
  const int taps_per = p.kt * p.kh * p.kw / parts;
  const int j_begin = split * taps_per * n_cb, j_end = j_begin + taps_per * n_cb;
  const long long w_tap_bytes = (long long)p.c_out * p.c_in * 2;

  const char* xsrc[kSlots];
  auto set_tap = [&](int tap) {
    const int a = tap / (p.kh * p.kw), bc = tap % (p.kh * p.kw);
    const int dt = a - (p.kt - 1), dy = bc / p.kw - (p.kh - 1) / 2, dx = bc % p.kw - (p.kw - 1) / 2;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) xsrc[i] = gather_row(p, px[i], xchunk[i], dt, dy, dx);
  };
  auto fetch = [&](int j, char* sw, char* sx) {
    const int tap = j / n_cb, cb = j % n_cb;
    const char* wb = uni(reinterpret_cast<const char*>(p.w) + tap * w_tap_bytes + cb * kRowBytes);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
      unsigned off = w_off[i];
      opaque(off);
      lds_dma16(wb + off, (lds_void*)(sw + (wave + kWaves * i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < kSlots; ++i)
      lds_dma16(xsrc[i] + cb * kRowBytes, (lds_void*)(sx + (wave + kWaves * i) * 1024));
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const char* sw, const char* sx) {
    const char* wa = sw + half_c * 64 * kRowBytes;
    const char* xb = sx + half_p * 64 * kRowBytes;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 av[4], bv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) av[k] = as_bf16x8(*reinterpret_cast<const uint4*>(wa + k * 16 * kRowBytes + rd[s]));
#pragma unroll
      for (int k = 0; k < 4; ++k) bv[k] = as_bf16x8(*reinterpret_cast<const uint4*>(xb + k * 16 * kRowBytes + rd[s]));
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    // operand reads of the second k-step overlap the first k-step's MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 16, 0);
  };

  set_tap(j_begin / n_cb);
  fetch(j_begin, sw0, sx0);
  for (int j = j_begin; j < j_end; j += 2) {
    // buffer 0 holds block j; block j+1 goes to buffer 1 meanwhile
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 1 < j_end) {
      if ((j + 1) % n_cb == 0) set_tap((j + 1) / n_cb);
      fetch(j + 1, sw1, sx1);
    }
    compute(sw0, sx0);
    if (j + 1 >= j_end) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 < j_end) {
      if ((j + 2) % n_cb == 0) set_tap((j + 2) / n_cb);
      fetch(j + 2, sw0, sx0);
    }
    compute(sw1, sx1);
  }

  // epilogue: lane holds output channels cout0 + 64 half_c + 16 a + 4 h + (0..3)
  // of pixel m0 + 64 half_p + 16 b + c16
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = m0 + half_p * 64 + b * 16 + c16;
    if (m >= n_pix) continue;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int co = cout0 + half_c * 64 + a * 16 + 4 * h;
      if (parts > 1) {
        *reinterpret_cast<float4*>(p.part + ((long long)split * n_pix + m) * p.c_out + co) =
            make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        continue;
      }
      const float4 bias = *reinterpret_cast<const float4*>(p.bias + co);
      const bf16x2 lo = {(__bf16)(acc[a][b][0] + bias.x), (__bf16)(acc[a][b][1] + bias.y)};
      const bf16x2 hi = {(__bf16)(acc[a][b][2] + bias.z), (__bf16)(acc[a][b][3] + bias.w)};
      *reinterpret_cast<uint2*>(p.y + (long long)m * p.c_out + co) =
          make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    }
  }
}

// Keep the last two input frames of the stream: frame f of the chunk is
// global frame k0 + f and goes to cache slot (k0 + f) mod 2 (frames
// first_frame .. frames-1; grid-stride over 16-byte units).
__device__ inline void copy_to_cache(const ConvParams& p, int first_frame) {
  const long long frame_u4 = (long long)p.height * p.width * p.c_in / 8;  // 16-byte units per frame
  const long long total = (p.frames - first_frame) * frame_u4;
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < total; u += (long long)gridDim.x * 256) {
    const int f = first_frame + (int)(u / frame_u4);
    const long long e = u % frame_u4;
    const uint4* src = reinterpret_cast<const uint4*>(p.x) + f * frame_u4 + e;
    uint4* dst = reinterpret_cast<uint4*>(p.cache) + ((p.k0 + f) & 1) * frame_u4 + e;
    *dst = *src;
  }
}

__global__ __launch_bounds__(256) void conv_cache_kernel(ConvParams p, int first_frame) {
  copy_to_cache(p, first_frame);
}

// After a call with split units: for each of their outputs, the sum of the
// partials plus bias, rounded to bf16 once (4 channels per thread), then the
// cache update (every conv workgroup has finished reading the cache by now).
__global__ __launch_bounds__(256) void conv_combine_kernel(ConvParams p, int first_frame) {
  const long long n_pix = (long long)p.frames * p.height * p.width;
  const int n_ct = p.c_out / kCout;
  const long long per_unit = (long long)kPix * kCout / 4;
  const long long total = (long long)(p.m_tiles * n_ct - p.whole) * per_unit;
  for (long long u = (long long)blockIdx.x * 256 + threadIdx.x; u < total; u += (long long)gridDim.x * 256) {
    const int unit = p.whole + (int)(u / per_unit);
    const int r = (int)(u % per_unit);
    const long long m = (long long)(unit / n_ct) * kPix + r / (kCout / 4);
    const int co = (unit % n_ct) * kCout + (r % (kCout / 4)) * 4;
    if (m >= n_pix) continue;
    float4 acc = *reinterpret_cast<const float4*>(p.bias + co);
    for (int s = 0; s < p.splits; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(p.part + (s * n_pix + m) * p.c_out + co);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const bf16x2 lo = {(__bf16)acc.x, (__bf16)acc.y};
    const bf16x2 hi = {(__bf16)acc.z, (__bf16)acc.w};
    *reinterpret_cast<uint2*>(p.y + m * p.c_out + co) =
        make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
  copy_to_cache(p, first_frame);
}

// Weights [C_out][C_in][taps] -> [taps][C_out][C_in]; bias bf16 -> float32
// (zero when absent); the zero row.
__global__ __launch_bounds__(256) void conv_pack_kernel(ConvPackParams p) {
  const long long n = (long long)p.c_out * p.c_in * p.taps;
  for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < n; e += (long long)gridDim.x * 256) {
    const int tap = (int)(e % p.taps);
    const long long oc = e / p.taps;  // o * C_in + ci
    const int ci = (int)(oc % p.c_in), o = (int)(oc / p.c_in);
    p.w_packed[((long long)tap * p.c_out + o) * p.c_in + ci] = p.weight[e];
  }
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < p.c_out) p.bias_out[t] = p.bias ? __uint_as_float((uint32_t)p.bias[t] << 16) : 0.f;
  if (t < p.zero_u4) reinterpret_cast<uint4*>(p.zero)[t] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_causal_conv(const ConvParams& p, hipStream_t s) {
  const int units = p.m_tiles * (p.c_out / kCout);
  const int split_units = units - p.whole;
  const int blocks_conv = p.whole + split_units * p.splits;
  hipLaunchKernelGGL(causal_conv_kernel, dim3(blocks_conv), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int first = p.frames > 2 ? p.frames - 2 : 0;
  long long work = (long long)(p.frames - first) * p.height * p.width * p.c_in / 8;  // cache units
  if (split_units > 0) {
    const long long out4 = (long long)split_units * kPix * kCout / 4;
    if (out4 > work) work = out4;
  }
  long long blocks = (work + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (split_units > 0)
    hipLaunchKernelGGL(conv_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, first);
  else
    hipLaunchKernelGGL(conv_cache_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, first);
  return hipGetLastError();
}

hipError_t launch_conv_pack(const ConvPackParams& p, hipStream_t s) {
  const long long n = (long long)p.c_out * p.c_in * p.taps;
  long long blocks = (n + 255) / 256;
  const long long need = ((p.c_out > p.zero_u4 ? p.c_out : p.zero_u4) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < need) blocks = need;
  hipLaunchKernelGGL(conv_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ckv
