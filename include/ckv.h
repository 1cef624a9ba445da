/*
 * ckv.h -- same-step chunk attention for an autoregressive, chunked video
 * diffusion transformer, on MI355X (gfx950).
 *
 * The method ("PhysisServe -- Wan2.2 5B" model card, "Inference profile"
 * table and the paragraph after it): a video is denoised chunk by chunk -- a
 * first chunk of F0 latent frames, then one-frame chunks -- with S denoising
 * steps per chunk.  At step s a chunk's queries attend to
 *   (1) the "sink": the first chunk's K/V from one extra clean (sigma = 0)
 *       pass, stored once;
 *   (2) the K/V that up to W preceding chunks recorded at the same step s
 *       (chunk 0 is present only as the sink, never duplicated);
 *   (3) the chunk's own K/V.
 * Queries and keys carry 3D rotary position embedding ("Learning Video
 * Generation from the Wan2.2 Source Code", Chapter 4, "3D RoPE": the head
 * dim is split into time/height/width bands of d-4(d/6), 2(d/6), 2(d/6)
 * dims and each adjacent pair is rotated by complex multiplication).
 *
 * Conventions for every call below
 *   - Tensors q, k, v, q_rot, out are bf16, contiguous [n_tokens][H][d]
 *     (token-major, then head, then head dim), n_tokens = F0*gh*gw for chunk
 *     0 and gh*gw for every later chunk.  Tokens are ordered frame-major,
 *     then patch row, then patch column.
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device and
 *     must be 16-byte aligned; the cache's arena must be on that device too
 *     (with several GPUs, make the arena's device current before each call:
 *     kernels launch on the current device).  The caller owns all device
 *     memory, including the cache arena; the library never allocates or
 *     frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously; no call synchronises the host.
 *     Inputs must stay valid until the stream has passed the call.
 *   - Errors are detected on the host before anything is enqueued; a call
 *     that returns an error other than CKV_E_HIP has changed no state and
 *     enqueued nothing.  CKV_E_HIP means a launch failed after validation.
 *   - A cache is not thread-safe, and its calls must be ordered on one
 *     stream (they share the cache's scratch area).  Distinct caches (e.g.
 *     one per prompt) are independent and may run on different streams
 *     concurrently.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ckv_status {
  CKV_OK = 0,
  CKV_E_INVALID = 1, /* bad argument: null/misaligned pointer, bad index, bad config */
  CKV_E_ORDER = 2,   /* chunk/step call out of the schedule's order               */
  CKV_E_STATE = 3,   /* cache state forbids the call (e.g. sink not built yet)    */
  CKV_E_ARENA = 4,   /* arena too small, null or not 256-byte aligned             */
  CKV_E_HIP = 5      /* a HIP launch or runtime call failed                       */
} ckv_status;

/* Step id of the first chunk's extra clean (sigma = 0) pass. */
#define CKV_STEP_SINK (-1)

/* Longest text context a layer stores ("Learning Video Generation from the
 * Wan2.2 Source Code", Chapter 3, "Where Did the Prompt Go?": the prompt
 * becomes up to 512 context vectors). */
#define CKV_MAX_TEXT_TOKENS 512

/* Model and schedule.  Layout is fixed (56 bytes) for foreign-function use. */
typedef struct ckv_config {
  int32_t num_layers;         /* caches kept per layer (e.g. 30)                      */
  int32_t num_steps;          /* denoising steps per chunk S (model card: 4)          */
  int32_t num_heads;          /* H (e.g. 24)                                          */
  int32_t head_dim;           /* d: 64 or 128                                         */
  int32_t grid_h;             /* patch rows of one latent frame (1280x704: 22)        */
  int32_t grid_w;             /* patch columns (1280x704: 40); grid_h*grid_w % 8 == 0 */
  int32_t first_chunk_frames; /* F0 (model card: 3)                                   */
  int32_t window_chunks;      /* W (model card: 18); ring capacity is W + 1 chunks    */
  int32_t max_chunks;         /* chunks per rollout, incl. the first (model card: 29) */
  int32_t reserved0;          /* must be 0                                            */
  double rope_theta;          /* RoPE base (10000)                                    */
  float softmax_scale;        /* 0 => 1/sqrt(head_dim)                                */
  int32_t reserved1;          /* must be 0                                            */
} ckv_config;

typedef struct ckv_cache ckv_cache; /* opaque; holds host state only */

/* One contiguous run of keys in a window, as the attention kernel reads it. */
typedef struct ckv_segment {
  int32_t kind;        /* 0 = the layer's sink area, 1 = a run of ring slots (step's ring) */
  int32_t first_slot;  /* ring slot of the run's first chunk (-1 for the sink area)        */
  int32_t chunk_first; /* chunk id of the run's first chunk (0 for the sink area)          */
  int32_t n_chunks;    /* chunks in the run                                                 */
  int32_t n_tokens;    /* keys in the run                                                   */
} ckv_segment;

/* Device bytes a cache with this config needs (angle tables + sinks + rings +
 * one text context per layer + split-key scratch), or 0 if the config is
 * invalid. */
size_t ckv_cache_bytes(const ckv_config* cfg);

/* Create a cache over a caller-owned device arena of at least
 * ckv_cache_bytes(cfg) bytes, 256-byte aligned.  Host-only: touches no device
 * memory.  The RoPE angle tables are built in the arena by a small kernel
 * enqueued on the stream of the cache's first device call (no host-to-device
 * copy, so that call does not block the host either).  Sink and ring layout inside the arena:
 *   sink  K [L][H][F0*gh*gw][d],  V transposed [L][H][d][F0*gh*gw];
 *   rings K [L][S][H][(W+1)*gh*gw][d], V transposed [L][S][H][d][(W+1)*gh*gw];
 *   text  K [L][H][CKV_MAX_TEXT_TOKENS][d], V transposed [L][H][d][CKV_MAX_TEXT_TOKENS].
 * Errors: CKV_E_INVALID (config), CKV_E_ARENA (arena). */
ckv_status ckv_cache_create(const ckv_config* cfg, void* device_arena, size_t arena_bytes,
                            ckv_cache** out);

/* Create a host-only "dry" cache: every call validates its arguments and the
 * schedule order and advances the state exactly as a real cache would, but
 * enqueues nothing and never dereferences tensor pointers (which must still
 * be non-null).  For planning and testing the schedule without a device. */
ckv_status ckv_cache_create_dry(const ckv_config* cfg, ckv_cache** out);

/* Start a new rollout: forget every appended chunk and the sink.  No device work. */
ckv_status ckv_cache_reset(ckv_cache* c);

/* Free the host state.  The arena remains the caller's. */
ckv_status ckv_cache_destroy(ckv_cache* c);

/* Per-step RoPE + K/V append (model card, paragraph after the "Inference
 * profile" table: later chunks read, at step s, the K/V that earlier chunks
 * stored at that same step s).  Rotates q and k by the
 * chunk's 3D positions (time = absolute latent frame: chunk 0 covers frames
 * 0..F0-1, chunk c >= 1 frame F0+c-1), writes the rotated q to q_rot, and
 * records the rotated k and v:
 *   chunk >= 1: into ring slot (chunk-1) mod (W+1) of (layer, step), evicting
 *               the chunk recorded W+1 chunks earlier.  Appends on one
 *               (layer, step) must come as chunk = 1, 2, 3, ... (CKV_E_ORDER)
 *               and need the layer's sink (CKV_E_STATE).
 *   chunk == 0: into the layer's sink area as scratch for chunk 0's own step;
 *               no later chunk reads it.  Not allowed once the sink is built
 *               (CKV_E_STATE).
 * 0 <= step < num_steps, 0 <= chunk < max_chunks, 0 <= layer < num_layers. */
ckv_status ckv_rope_append(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                           const void* q, const void* k, const void* v, void* q_rot,
                           void* stream);

/* The first chunk's extra clean (sigma = 0) pass (model card, paragraph after
 * the "Inference profile" table: chunk 0 gets one more forward pass whose K/V
 * become the persistent sink).  Rotates q and k of
 * chunk 0 (frames 0..F0-1), writes q_rot, and stores the rotated k and v as
 * the layer's sink, shared by every step.  Once per layer per rollout
 * (CKV_E_STATE on a second call before ckv_cache_reset). */
ckv_status ckv_sink_build(ckv_cache* c, int32_t layer, const void* q, const void* k,
                          const void* v, void* q_rot, void* stream);

/* The same two calls with the QK-Norm in front ("Learning Video Generation
 * from the Wan2.2 Source Code", Chapter 4, "3D RoPE" detail paragraph: q and k
 * each pass an RMSNorm after their linear layers).  q and k are the raw
 * projections [n_tokens][H][d] bf16; each token's whole projected vector (all
 * H*d values) is divided by sqrt(mean of its squares + eps) and multiplied
 * channel-wise by q_gain / k_gain, rounded to bf16 (the norm's output
 * precision), and then rotated and stored exactly as ckv_rope_append /
 * ckv_sink_build do.  v is not normalised.
 *   q_gain, k_gain: device float32 [H*d] (channel h*d + i is head h, dim i),
 *                   16-byte aligned, read during the call (keep them alive
 *                   until the stream passes it).
 *   eps: finite and > 0 (else CKV_E_INVALID, nothing launched).
 * Order and state rules and all other errors are those of the plain calls. */
ckv_status ckv_norm_rope_append(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                                const void* q, const void* k, const void* v,
                                const float* q_gain, const float* k_gain, float eps,
                                void* q_rot, void* stream);
ckv_status ckv_norm_sink_build(ckv_cache* c, int32_t layer, const void* q, const void* k,
                               const void* v, const float* q_gain, const float* k_gain, float eps,
                               void* q_rot, void* stream);

/* Chunk attention ("PhysisServe -- Wan2.2 5B" model card, "Inference
 * profile" table, KV-history row, and the paragraph after the table: a
 * chunk's queries see the clean first-chunk sink, at most W earlier chunks'
 * K/V from the same denoising step, chunk 0 never twice, and its own K/V):
 * out = softmax(scale * q_rot K_win^T) V_win per head, no
 * mask, with K_win/V_win gathered in place from
 *   chunk == 0, step in [0,S): the chunk's own step-`step` K/V (needs that
 *               append to be the last write to the sink area; CKV_E_STATE);
 *   chunk == 0, step == CKV_STEP_SINK: the sink itself (the clean pass's
 *               self-attention; needs the sink);
 *   chunk >= 1: [sink | chunks max(1,chunk-W) .. chunk-1 at this step | own],
 *               needing `chunk` to be the last append on (layer, step)
 *               (CKV_E_ORDER).
 * q_rot is [n_tokens][H][d] as written by the matching append/sink call;
 * out is [n_tokens][H][d] bf16.  The softmax is accumulated in fp32. */
ckv_status ckv_chunk_attention(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                               const void* q_rot, void* out, void* stream);

/* The same chunk attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): identical arguments, checks, kernels and results, but the
 * partials (fp16 outputs, float32 log-sum-exps) of a key-split call live in the library's own static
 * device array (CKV_STATIC_SCRATCH_BYTES per GPU, held until the process
 * ends) instead of the cache arena.  Allocates nothing.  Every call on one
 * GPU shares that array: calls that overlap in time on one GPU (two streams,
 * two caches) race, so order them on one stream.  A call whose partials
 * would exceed the array returns CKV_E_INVALID and enqueues nothing (the
 * split policy keeps every call of a valid config within it). */
#define CKV_STATIC_SCRATCH_BYTES ((size_t)2 * 256 * 128 * (128 * 2 + 4))
ckv_status ckv_chunk_attention_static(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                                      const void* q_rot, void* out, void* stream);

/* Store one layer's text context for cross-attention ("Learning Video
 * Generation from the Wan2.2 Source Code", Chapter 3, "Where Did the Prompt
 * Go?": the context, trimmed to the prompt's real length, is the key/value of
 * every layer's cross-attention and never changes during a rollout).
 * k_text, v_text: [n_text][H][d] bf16 device tensors, the layer's projected
 * context keys and values (no rotation), read during the call.
 * 1 <= n_text <= CKV_MAX_TEXT_TOKENS, 0 <= layer < num_layers (else
 * CKV_E_INVALID).  Replaces any context stored for the layer; cleared by
 * ckv_cache_reset.  The arena holds one context per layer
 * (ckv_cache_bytes includes it). */
ckv_status ckv_text_store(ckv_cache* c, int32_t layer, const void* k_text, const void* v_text,
                          int32_t n_text, void* stream);

/* Cross-attention of one chunk's video tokens to the layer's stored context
 * (same chapter; the block's cross-attention takes the video tokens as
 * queries): out = softmax(scale * q K_text^T) V_text per head over the n_text
 * stored rows, no mask, no rotation.  q and out are [tokens(chunk)][H][d]
 * bf16 (2640 rows for chunk 0, h*w per later chunk).  CKV_E_STATE if the
 * layer has no context; independent of the ring schedule. */
ckv_status ckv_cross_attention(ckv_cache* c, int32_t layer, int32_t chunk, const void* q,
                               void* out, void* stream);

/* Host-only: the window (layer, step, chunk) attends to (model card,
 * "Inference profile" table, KV-history row: the sink plus at most W of the
 * most recent earlier chunks, chunk 0 only as the sink), as <= 3 segments in
 * key order (sink area, then up to two runs of ring slots; the last run ends
 * with the chunk itself).  Depends only on the config.  *n_segs receives the
 * count; CKV_E_INVALID if max_segs is too small or an index is out of range. */
ckv_status ckv_window(const ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                      ckv_segment* segs, int32_t max_segs, int32_t* n_segs);

/* Host-only: the ring slot chunk >= 1 occupies on any (layer, step) ring. */
ckv_status ckv_ring_slot(const ckv_cache* c, int32_t chunk, int32_t* slot);

/* Copy the stored rotated K and V of (layer, step, chunk) out to caller
 * buffers k_out, v_out [n_tokens][H][d] bf16 (for checking).  chunk == 0
 * with step == CKV_STEP_SINK copies the sink; chunk == 0 with a step copies
 * the sink area if it holds that step's K/V; chunk >= 1 must still be live in
 * the (layer, step) ring (CKV_E_STATE otherwise). */
ckv_status ckv_debug_copy_kv(const ckv_cache* c, int32_t layer, int32_t step, int32_t chunk,
                             void* k_out, void* v_out, void* stream);

/* Key splits the next attention over `n_keys` keys with `n_queries` queries
 * would use (1 = no split), for reporting.  Host-only. */
int32_t ckv_attention_splits(const ckv_cache* c, int32_t n_queries, int32_t n_keys);

/* Static, human-readable name of a status code. */
const char* ckv_status_string(ckv_status st);

#ifdef __cplusplus
}
#endif

#endif /* CKV_H */
