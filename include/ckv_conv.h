/*
 * ckv_conv.h -- streaming causal 3D convolution with a temporal cache, the
 * chunked-cache workload of the video VAE decoder, on MI355X (gfx950).
 *
 * The operation ("Learning Video Generation from the Wan2.2 Source Code",
 * Chapter 2, "Causal Convolution and Streaming Inference"): a Conv3d whose
 * time padding sits entirely in front of the sequence (kt - 1 frames, none
 * behind), so every output frame depends only on its own and earlier input
 * frames; the spatial padding is symmetric ((kh-1)/2, (kw-1)/2).  A video is
 * fed chunk by chunk: the last CACHE_T = 2 input frames seen so far are kept
 * and stand in front of the next chunk in place of that much zero padding,
 * which gives exactly the whole-video result, with memory independent of
 * the video's length.
 *
 *   y[t][i][j][o] = bias[o] + sum_{a,b,c,ci} W[o][ci][a][b][c]
 *                   * x[t + a - (kt-1)][i + b - (kh-1)/2][j + c - (kw-1)/2][ci]
 *   with x = 0 outside the video (before its first frame, outside the grid)
 *   and t counted over the whole stream since the last reset.
 *
 * Conventions (as in ckv.h; status codes are ckv_status)
 *   - Activations x, y are bf16, contiguous [frames][H][W][C] (channels last:
 *     the same data as PyTorch's [C][T][H][W] tensor of one video, in the
 *     channels_last_3d order).  Weights are bf16 in Conv3d's own layout
 *     [C_out][C_in][kt][kh][kw]; bias is bf16 [C_out] or NULL (zero).
 *     Accumulation is float32; y is rounded to bf16 (nearest even) once.
 *   - Device pointers on the current HIP device (the state arena's device),
 *     16-byte aligned; the caller owns all device memory,
 *     including the state arena (ckv_conv_bytes); the library never
 *     allocates, frees or synchronises.  x and y must not overlap.
 *   - `stream` is a hipStream_t passed as void*; calls on one state object
 *     must be ordered on one stream (each call reads the cache the previous
 *     call left).  Errors other than CKV_E_HIP are found on the host before
 *     anything is enqueued and change no state.
 */
#ifndef CKV_CONV_H
#define CKV_CONV_H

#include <stddef.h>
#include <stdint.h>

#include "ckv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Input frames kept between chunks (the page's CACHE_T). */
#define CKV_CONV_CACHE_T 2

typedef struct ckv_conv ckv_conv; /* opaque host-side state */

typedef struct ckv_conv_config {
  int32_t height, width;    /* frame grid H x W, each >= 1                           */
  int32_t in_channels;      /* C_in, a multiple of 64                                 */
  int32_t out_channels;     /* C_out, a multiple of 128                               */
  int32_t kt, kh, kw;       /* kernel: kt in 1..3 (<= CACHE_T + 1), kh and kw in {1,3} */
  int32_t max_frames;       /* largest chunk a call may pass, >= 1                    */
} ckv_conv_config;

/* Arena bytes for one layer's state (packed weights, bias, the 2-frame
 * cache, a zero row, and float32 partials of a split call: kt * max_frames
 * * H * W * C_out floats when kt > 1); 0 if the config is invalid. */
size_t ckv_conv_bytes(const ckv_conv_config* cfg);

/* Create a state object over a caller-owned device arena (>= ckv_conv_bytes,
 * 256-byte aligned).  Host-only: nothing is enqueued. */
ckv_status ckv_conv_create(const ckv_conv_config* cfg, void* device_arena, size_t arena_bytes,
                           ckv_conv** out);

/* Host-only state for tests of the argument checks (no device, no arena);
 * ckv_causal_conv and ckv_conv_set_weights validate and then return CKV_OK
 * without enqueueing. */
ckv_status ckv_conv_create_dry(const ckv_conv_config* cfg, ckv_conv** out);

/* Load the layer's weights: packs weight [C_out][C_in][kt][kh][kw] bf16 into
 * the arena's tap-major layout, converts bias (bf16 [C_out] or NULL) to
 * float32, and zeroes the arena's zero row.  Must precede the first
 * ckv_causal_conv; may be called again (new weights) at any time between
 * calls.  The inputs may be freed once the stream has passed this call. */
ckv_status ckv_conv_set_weights(ckv_conv* c, const void* weight, const void* bias, void* stream);

/* Start a new video: the next call sees no history (zeros before its first
 * frame).  Host-only; nothing is enqueued. */
ckv_status ckv_conv_reset(ckv_conv* c);

/* One chunk: y = causal conv of x with the cached history in front, then the
 * cache keeps the last CACHE_T input frames of the stream.  x [frames][H][W]
 * [C_in], y [frames][H][W][C_out], 1 <= frames <= max_frames.
 * CKV_E_STATE if no weights were set. */
ckv_status ckv_causal_conv(ckv_conv* c, const void* x, int32_t frames, void* y, void* stream);

/* Frames consumed since the last reset (the global index of the next
 * chunk's first frame). */
int64_t ckv_conv_position(const ckv_conv* c);

/* How a call of `frames` frames runs its (pixel tile, channel tile) units:
 * the first *whole_units of them (if whole_units is not NULL) over all taps,
 * every later one as `return value` parts, part s summing the taps of time
 * offset s (float32 partials, summed with the bias by a second kernel).
 * Units split when the call alone would leave CUs idle, or when they form a
 * last, partly filled round of two workgroups per CU.  The device's CU count
 * is read on the first ckv_causal_conv; before that (and for a dry state)
 * 256 is assumed.  Returns 0 for invalid arguments. */
int32_t ckv_conv_splits(const ckv_conv* c, int32_t frames, int32_t* whole_units);

ckv_status ckv_conv_destroy(ckv_conv* c);

#ifdef __cplusplus
}
#endif

#endif /* CKV_CONV_H */
