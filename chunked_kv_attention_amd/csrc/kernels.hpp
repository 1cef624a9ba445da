// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace ckv {

typedef uint16_t bf16_t;  // raw bf16 storage

// Rotate q and k of one chunk by 3D RoPE; write q_rot and the K/V store.
struct RopeAppendParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* q_rot;
  bf16_t* k_dst;             // [H][rows][d]: the chunk's first row, head 0
  bf16_t* vt_dst;            // [H][d][cols]: the chunk's first column, head 0
  long long k_head_stride;   // elements between heads in k_dst
  long long vt_head_stride;  // elements between heads in vt_dst
  int vt_row_stride;         // elements between head-dim rows in vt_dst
  int n_tokens;
  int num_heads;
  int first_frame;           // absolute latent frame of the chunk's first frame
  int grid_h, grid_w;
  const float* cos_sin;      // [frames][Dt/2] | [grid_h][Dh/2] | [grid_w][Dw/2] float2 (cos, sin)
  int n_frames_table;
  // QK-Norm (optional; null gains = q and k used as given): each token's q
  // and k are first divided by the root of the mean of squares of their
  // whole projected vector (H * d values) plus eps, scaled by a per-channel
  // gain, rounded to bf16, and only then rotated.
  const float* q_gain;       // [H * d] or null
  const float* k_gain;       // [H * d] or null
  float eps;
};

// RoPE angle tables of a cache: float2 (cos, sin) per band pair and position,
// time band [frames][band_t/2], then height [grid_h][band_h/2], then width
// [grid_w][band_w/2], from float64 angles rounded once to float32.
struct RopeTableParams {
  float2* out;
  int frames, grid_h, grid_w;
  int band_t, band_h, band_w;  // widths in dims
  double theta;
};

// The text context of one layer into the attention store: K rows
// [H][max_text][d] and V^T [H][d][max_text], V^T columns past n_text zeroed.
struct TextStoreParams {
  const bf16_t* k;           // [n_text][H][d]
  const bf16_t* v;           // [n_text][H][d]
  bf16_t* k_dst;
  bf16_t* vt_dst;
  int n_text, max_text, num_heads;
};

// Up to three runs of keys, in key order; run r holds keys [end[r-1], end[r]).
struct AttnParams {
  const bf16_t* q;           // [nq][H][d]
  bf16_t* out;               // [nq][H][d]
  const bf16_t* k[3];        // run base, head 0: [rows][d]
  const bf16_t* vt[3];       // run base, head 0: [d][cols]
  long long k_head_stride[3];
  long long vt_head_stride[3];
  int vt_row_stride[3];
  int seg_end[3];            // cumulative key counts; unused runs repeat n_keys
  int n_queries;
  int n_keys;
  int num_heads;
  int n_splits;              // key splits; 1 writes `out` directly
  int q_tiles;               // ceil(nq / query tile)
  int key_tiles;             // ceil(n_keys / key tile)
  float scale_log2;          // softmax scale * log2(e)
  uint16_t* part_o;          // [n_splits][nq][H][d] fp16 (split > 1); n_splits*nq*H <= kAttnScratchRows
  float* part_lse;           // [n_splits][nq][H]   log2-domain LSE (split > 1)
};

struct CopyKVParams {
  const bf16_t* k_src;  // [H][rows][d] at the chunk's first row
  const bf16_t* vt_src; // [H][d][cols] at the chunk's first column
  long long k_head_stride, vt_head_stride;
  int vt_row_stride;
  int n_tokens, num_heads;
  bf16_t* k_out;        // [n][H][d]
  bf16_t* v_out;        // [n][H][d]
};

// Streaming causal 3D convolution of one chunk (implicit GEMM).  Tap order
// is Conv3d's (a, b, c) over (kt, kh, kw), a slowest.
struct ConvParams {
  const bf16_t* x;           // [frames][H][W][C_in]
  bf16_t* y;                 // [frames][H][W][C_out]
  const bf16_t* w;           // packed [taps][C_out][C_in]
  const float* bias;         // [C_out]
  bf16_t* cache;             // [2][H][W][C_in]: global frame g in slot g mod 2
  const bf16_t* zero;        // >= C_in zeros (source of out-of-video taps)
  long long k0;              // global index of the chunk's first frame
  int frames, height, width, c_in, c_out, kt, kh, kw;
  int m_tiles;               // ceil(frames * H * W / kConvPixelTile)
  // Units (pixel tile, channel tile) 0 .. whole-1 run over all taps; each
  // later unit runs as `splits` parts, part s summing the taps of time offset
  // s only and writing float32 partials (splits = 1: no split units).
  int whole;
  int splits;                // 1, or kt
  float* part;               // [splits][frames * H * W][C_out] float32 (split units)
};

// Weights [C_out][C_in][taps] -> [taps][C_out][C_in], bias bf16 -> float32.
struct ConvPackParams {
  const bf16_t* weight;
  const bf16_t* bias;        // or null (zero bias)
  bf16_t* w_packed;
  float* bias_out;
  bf16_t* zero;              // zero_u4 16-byte units set to 0
  int c_out, c_in, taps, zero_u4;
};

constexpr int kConvPixelTile = 128;    // output pixels per workgroup
constexpr int kConvChannelTile = 128;  // output channels per workgroup

constexpr int kAttnQueryTile = 128;  // query rows per workgroup
constexpr int kAttnKeyTile = 64;     // keys per LDS tile
constexpr int kAttnMaxSplits = 32;   // most key splits of one call
// Rows (query, head) of partials (an fp16 output row and a float32
// log-sum-exp each) the split scratch holds: every split
// workgroup of a call owns one query tile of one head, and a call is split
// only while its workgroups fit the chip's 2-per-CU slots once, so 2 x 256
// CUs x 128 rows bound every split call on MI355X.
constexpr int kAttnScratchRows = 2 * 256 * kAttnQueryTile;

// Bytes of the library's static split scratch (fp16 partial outputs at
// head_dim 128 plus float32 log-sum-exps for every scratch row), and its
// device address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)kAttnScratchRows * (128 * 2 + 4);
hipError_t static_scratch(void** ptr);

hipError_t launch_rope_append(const RopeAppendParams& p, int head_dim, hipStream_t s);
hipError_t launch_rope_table(const RopeTableParams& p, hipStream_t s);
hipError_t launch_text_store(const TextStoreParams& p, int head_dim, hipStream_t s);
hipError_t launch_chunk_attention(const AttnParams& p, int head_dim, hipStream_t s);
hipError_t launch_copy_kv(const CopyKVParams& p, int head_dim, hipStream_t s);
hipError_t launch_causal_conv(const ConvParams& p, hipStream_t s);
hipError_t launch_conv_pack(const ConvPackParams& p, hipStream_t s);

}  // namespace ckv
