// C-ABI of the same-step chunk attention library (declared in include/ckv.h).
//
// Host responsibilities: validate every call against the config and the
// schedule (ring_index.hpp), lay out the caller's arena, have the RoPE angle
// tables built once on the device (float64, rounded once to float32), turn a
// window into at most three key runs, pick the key-split count, and launch
// the kernels on the caller's stream.  Nothing here allocates device memory,
// copies from the host or synchronises.
#include "ckv.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.hpp"
#include "ring_index.hpp"

namespace {

using ckv::bf16_t;

constexpr size_t kAlign = 256;
constexpr int kMaxSplits = ckv::kAttnMaxSplits;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Bands {
  int t, h, w;  // widths in dims
};
Bands bands_of(int d) { return Bands{d - 4 * (d / 6), 2 * (d / 6), 2 * (d / 6)}; }

struct Layout {
  int n1 = 0, n0 = 0, ring_rows = 0, frames_table = 0;
  size_t tables_off = 0, tables_bytes = 0;
  size_t sink_off = 0, sink_layer_bytes = 0;
  size_t ring_off = 0, ring_bytes = 0;  // per (layer, step)
  size_t part_o_off = 0, part_lse_off = 0;
  size_t text_off = 0, text_layer_bytes = 0;  // per layer: context K [H][max][d], V^T [H][d][max]
  size_t total = 0;
};

bool config_ok(const ckv_config* c) {
  if (!c) return false;
  if (c->num_layers <= 0 || c->num_steps <= 0 || c->num_heads <= 0) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->grid_h <= 0 || c->grid_w <= 0 || ((long long)c->grid_h * c->grid_w) % 8 != 0) return false;
  if ((long long)c->grid_h * c->grid_w > (1 << 20)) return false;
  if (c->first_chunk_frames <= 0 || c->window_chunks < 0 || c->max_chunks <= 0) return false;
  if (c->reserved0 != 0 || c->reserved1 != 0) return false;
  if (!(c->rope_theta > 1.0) || !std::isfinite(c->rope_theta)) return false;
  if (!(c->softmax_scale >= 0.0f) || !std::isfinite(c->softmax_scale)) return false;
  // Key and element counts must stay inside 32-bit kernel indexing.
  const long long n1 = (long long)c->grid_h * c->grid_w;
  const long long ring_rows = (long long)(c->window_chunks + 1) * n1;
  const long long keys = (long long)c->first_chunk_frames * n1 + ring_rows;
  if (keys >= (1LL << 30) || ring_rows * c->head_dim >= (1LL << 31)) return false;
  if ((long long)c->first_chunk_frames * n1 * c->num_heads * c->head_dim >= (1LL << 31)) return false;
  return true;
}

Layout layout_of(const ckv_config* c) {
  Layout L;
  const Bands b = bands_of(c->head_dim);
  L.n1 = c->grid_h * c->grid_w;
  L.n0 = c->first_chunk_frames * L.n1;
  L.ring_rows = (c->window_chunks + 1) * L.n1;
  L.frames_table = c->first_chunk_frames + c->max_chunks - 1;
  const size_t H = c->num_heads, d = c->head_dim;
  size_t off = 0;
  L.tables_off = off;
  L.tables_bytes =
      sizeof(float) * 2 * ((size_t)L.frames_table * (b.t / 2) + (size_t)c->grid_h * (b.h / 2) + (size_t)c->grid_w * (b.w / 2));
  off = align_up(off + L.tables_bytes);
  L.sink_off = off;
  L.sink_layer_bytes = align_up(2 * H * L.n0 * d * sizeof(bf16_t));
  off += L.sink_layer_bytes * c->num_layers;
  L.ring_off = off;
  L.ring_bytes = align_up(2 * H * (size_t)L.ring_rows * d * sizeof(bf16_t));
  off += L.ring_bytes * c->num_layers * c->num_steps;
  L.part_o_off = off;
  off = align_up(off + sizeof(uint16_t) * ckv::kAttnScratchRows * d);
  L.part_lse_off = off;
  off = align_up(off + sizeof(float) * ckv::kAttnScratchRows);
  L.text_off = off;
  L.text_layer_bytes = align_up(2 * H * (size_t)CKV_MAX_TEXT_TOKENS * d * sizeof(bf16_t));
  off += L.text_layer_bytes * c->num_layers;
  L.total = off;
  return L;
}

}  // namespace

struct ckv_cache {
  ckv_config cfg;
  bool dry;
  char* arena;
  size_t arena_bytes;
  Layout L;
  ckv::Schedule sched;
  bool tables_built;  // the angle tables are built in the arena on the first device call
  int num_cus;
  std::vector<int> text_len;  // per layer: context rows stored (0 = none)

  ckv_cache(const ckv_config& c, bool is_dry, char* a, size_t bytes)
      : cfg(c), dry(is_dry), arena(a), arena_bytes(bytes), L(layout_of(&c)),
        sched(c.num_layers, c.num_steps, c.window_chunks, c.max_chunks, c.first_chunk_frames * c.grid_h * c.grid_w,
              c.grid_h * c.grid_w),
        tables_built(false), num_cus(0), text_len(c.num_layers, 0) {}

  bf16_t* sink_k(int layer) const { return (bf16_t*)(arena + L.sink_off + L.sink_layer_bytes * layer); }
  bf16_t* sink_vt(int layer) const { return sink_k(layer) + (size_t)cfg.num_heads * L.n0 * cfg.head_dim; }
  bf16_t* ring_k(int layer, int step) const {
    return (bf16_t*)(arena + L.ring_off + L.ring_bytes * ((size_t)layer * cfg.num_steps + step));
  }
  bf16_t* ring_vt(int layer, int step) const {
    return ring_k(layer, step) + (size_t)cfg.num_heads * L.ring_rows * cfg.head_dim;
  }
  bf16_t* text_k(int layer) const { return (bf16_t*)(arena + L.text_off + L.text_layer_bytes * layer); }
  bf16_t* text_vt(int layer) const { return text_k(layer) + (size_t)cfg.num_heads * CKV_MAX_TEXT_TOKENS * cfg.head_dim; }
  float scale() const { return cfg.softmax_scale > 0 ? cfg.softmax_scale : 1.0f / std::sqrt((float)cfg.head_dim); }
  int tokens(int chunk) const { return chunk == 0 ? L.n0 : L.n1; }
};

namespace {

ckv_status to_status(ckv::Check c) {
  switch (c) {
    case ckv::Check::kOk: return CKV_OK;
    case ckv::Check::kInvalid: return CKV_E_INVALID;
    case ckv::Check::kOrder: return CKV_E_ORDER;
    case ckv::Check::kState: return CKV_E_STATE;
  }
  return CKV_E_INVALID;
}

bool ptr_ok(const void* p) { return p != nullptr && ((uintptr_t)p % 16) == 0; }

ckv_status ensure_device(ckv_cache* c, hipStream_t s) {
  if (c->num_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CKV_E_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return CKV_E_HIP;
    c->num_cus = cus > 0 ? cus : 256;
  }
  if (!c->tables_built) {
    // 3D RoPE angle tables ("Learning Video Generation from the Wan2.2 Source
    // Code", Chapter 4, "3D RoPE"): per band of width D, pair j rotates by
    // pos * theta^(-2j/D); built by a kernel on the call's stream, so the
    // first call stays asynchronous like every other.
    const Bands b = bands_of(c->cfg.head_dim);
    ckv::RopeTableParams t;
    t.out = (float2*)(c->arena + c->L.tables_off);
    t.frames = c->L.frames_table;
    t.grid_h = c->cfg.grid_h;
    t.grid_w = c->cfg.grid_w;
    t.band_t = b.t;
    t.band_h = b.h;
    t.band_w = b.w;
    t.theta = c->cfg.rope_theta;
    if (ckv::launch_rope_table(t, s) != hipSuccess) return CKV_E_HIP;
    c->tables_built = true;
  }
  return CKV_OK;
}

int splits_for(int num_cus, int heads, int n_queries, int n_keys) {
  const int q_tiles = (n_queries + ckv::kAttnQueryTile - 1) / ckv::kAttnQueryTile;
  const int key_tiles = (n_keys + ckv::kAttnKeyTile - 1) / ckv::kAttnKeyTile;
  const long long units = (long long)q_tiles * heads;
  const long long slots = 2LL * (num_cus > 0 ? num_cus : 256);  // two workgroups per CU
  long long p = slots / (units > 0 ? units : 1);
  if (p > kMaxSplits) p = kMaxSplits;
  // keep >= 8 key tiles per split: below that the merge kernel and the
  // partials cost more than the idle CUs of an unsplit call (measured: an
  // 880 x 512 cross-attention takes 16 us unsplit, 26 us split in two)
  if (p > key_tiles / 8) p = key_tiles / 8;
  // the partials of every split must fit the scratch rows
  const long long rows = (long long)n_queries * heads;
  if (p * rows > ckv::kAttnScratchRows) p = ckv::kAttnScratchRows / rows;
  return p < 1 ? 1 : (int)p;
}

// Optional QK-Norm of an append / sink build: gains over the projected
// vector (H * d floats each) and eps; q_gain == nullptr means no norm.
struct QkNorm {
  const float* q_gain = nullptr;
  const float* k_gain = nullptr;
  float eps = 0.f;
};

bool norm_ok(const QkNorm& n) {
  return n.q_gain && n.k_gain && ((uintptr_t)n.q_gain % 16) == 0 && ((uintptr_t)n.k_gain % 16) == 0 &&
         std::isfinite(n.eps) && n.eps > 0.f;
}

ckv_status rope_store(ckv_cache* c, int chunk, bf16_t* k_dst, bf16_t* vt_dst, long long k_hs, long long vt_hs,
                      int vt_row, const void* q, const void* k, const void* v, void* q_rot, hipStream_t s,
                      const QkNorm& norm = QkNorm()) {
  ckv::RopeAppendParams p;
  p.q_gain = norm.q_gain;
  p.k_gain = norm.k_gain;
  p.eps = norm.eps;
  p.q = (const bf16_t*)q;
  p.k = (const bf16_t*)k;
  p.v = (const bf16_t*)v;
  p.q_rot = (bf16_t*)q_rot;
  p.k_dst = k_dst;
  p.vt_dst = vt_dst;
  p.k_head_stride = k_hs;
  p.vt_head_stride = vt_hs;
  p.vt_row_stride = vt_row;
  p.n_tokens = c->tokens(chunk);
  p.num_heads = c->cfg.num_heads;
  p.first_frame = chunk == 0 ? 0 : c->cfg.first_chunk_frames + chunk - 1;
  p.grid_h = c->cfg.grid_h;
  p.grid_w = c->cfg.grid_w;
  p.cos_sin = (const float*)(c->arena + c->L.tables_off);
  p.n_frames_table = c->L.frames_table;
  return ckv::launch_rope_append(p, c->cfg.head_dim, s) == hipSuccess ? CKV_OK : CKV_E_HIP;
}

ckv_status append_impl(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q, const void* k,
                       const void* v, void* q_rot, void* stream, const QkNorm& norm) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(q_rot)) return CKV_E_INVALID;
  ckv_status st = to_status(c->sched.check_append(layer, step, chunk));
  if (st != CKV_OK) return st;
  if (!c->dry) {
    hipStream_t s = (hipStream_t)stream;
    if ((st = ensure_device(c, s)) != CKV_OK) return st;
    const size_t d = c->cfg.head_dim;
    if (chunk == 0) {
      st = rope_store(c, 0, c->sink_k(layer), c->sink_vt(layer), (long long)c->L.n0 * d, (long long)d * c->L.n0,
                      c->L.n0, q, k, v, q_rot, s, norm);
    } else {
      const int slot = c->sched.slot_of(chunk);
      st = rope_store(c, chunk, c->ring_k(layer, step) + (size_t)slot * c->L.n1 * d,
                      c->ring_vt(layer, step) + (size_t)slot * c->L.n1, (long long)c->L.ring_rows * d,
                      (long long)d * c->L.ring_rows, c->L.ring_rows, q, k, v, q_rot, s, norm);
    }
    if (st != CKV_OK) return st;
  }
  c->sched.commit_append(layer, step, chunk);
  return CKV_OK;
}

ckv_status sink_impl(ckv_cache* c, int32_t layer, const void* q, const void* k, const void* v, void* q_rot,
                     void* stream, const QkNorm& norm) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(q_rot)) return CKV_E_INVALID;
  ckv_status st = to_status(c->sched.check_sink_build(layer));
  if (st != CKV_OK) return st;
  if (!c->dry) {
    hipStream_t s = (hipStream_t)stream;
    if ((st = ensure_device(c, s)) != CKV_OK) return st;
    const size_t d = c->cfg.head_dim;
    st = rope_store(c, 0, c->sink_k(layer), c->sink_vt(layer), (long long)c->L.n0 * d, (long long)d * c->L.n0,
                    c->L.n0, q, k, v, q_rot, s, norm);
    if (st != CKV_OK) return st;
  }
  c->sched.commit_sink_build(layer);
  return CKV_OK;
}

ckv_status attention_impl(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q_rot, void* out,
                          void* stream, bool static_scratch) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(q_rot) || !ptr_ok(out)) return CKV_E_INVALID;
  ckv_status st = to_status(c->sched.check_attention(layer, step, chunk));
  if (st != CKV_OK) return st;
  if (c->dry) return CKV_OK;
  hipStream_t s = (hipStream_t)stream;
  if ((st = ensure_device(c, s)) != CKV_OK) return st;

  ckv::Segment segs[3];
  const int nseg = c->sched.window(chunk, segs);
  const long long d = c->cfg.head_dim;
  ckv::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  int end = 0;
  for (int i = 0; i < 3; ++i) {
    if (i < nseg) {
      const ckv::Segment& g = segs[i];
      if (g.kind == 0) {
        p.k[i] = c->sink_k(layer);
        p.vt[i] = c->sink_vt(layer);
        p.k_head_stride[i] = (long long)c->L.n0 * d;
        p.vt_head_stride[i] = d * c->L.n0;
        p.vt_row_stride[i] = c->L.n0;
      } else {
        p.k[i] = c->ring_k(layer, step) + (size_t)g.first_slot * c->L.n1 * d;
        p.vt[i] = c->ring_vt(layer, step) + (size_t)g.first_slot * c->L.n1;
        p.k_head_stride[i] = (long long)c->L.ring_rows * d;
        p.vt_head_stride[i] = d * c->L.ring_rows;
        p.vt_row_stride[i] = c->L.ring_rows;
      }
      end += g.n_tokens;
    } else {
      p.k[i] = p.k[0];
      p.vt[i] = p.vt[0];
      p.k_head_stride[i] = p.k_head_stride[0];
      p.vt_head_stride[i] = p.vt_head_stride[0];
      p.vt_row_stride[i] = p.vt_row_stride[0];
    }
    p.seg_end[i] = end;
  }
  p.q = (const bf16_t*)q_rot;
  p.out = (bf16_t*)out;
  p.n_queries = c->tokens(chunk);
  p.n_keys = end;
  p.num_heads = c->cfg.num_heads;
  p.n_splits = splits_for(c->num_cus, c->cfg.num_heads, p.n_queries, p.n_keys);
  p.q_tiles = (p.n_queries + ckv::kAttnQueryTile - 1) / ckv::kAttnQueryTile;
  p.key_tiles = (p.n_keys + ckv::kAttnKeyTile - 1) / ckv::kAttnKeyTile;
  p.scale_log2 = c->scale() * 1.4426950408889634f;
  if (static_scratch) {
    // the library's own array: partial outputs, then the log-sum-exps
    const size_t rows = (size_t)p.n_splits * p.n_queries * p.num_heads;
    if (p.n_splits > 1 && rows * (d * sizeof(uint16_t) + sizeof(float)) > ckv::kStaticScratchBytes)
      return CKV_E_INVALID;
    void* base = nullptr;
    if (ckv::static_scratch(&base) != hipSuccess) return CKV_E_HIP;
    p.part_o = (uint16_t*)base;
    p.part_lse = (float*)((char*)base + rows * d * sizeof(uint16_t));
  } else {
    p.part_o = (uint16_t*)(c->arena + c->L.part_o_off);
    p.part_lse = (float*)(c->arena + c->L.part_lse_off);
  }
  return ckv::launch_chunk_attention(p, c->cfg.head_dim, s) == hipSuccess ? CKV_OK : CKV_E_HIP;
}

}  // namespace

extern "C" {

size_t ckv_cache_bytes(const ckv_config* cfg) { return config_ok(cfg) ? layout_of(cfg).total : 0; }

ckv_status ckv_cache_create(const ckv_config* cfg, void* device_arena, size_t arena_bytes, ckv_cache** out) {
  if (!out) return CKV_E_INVALID;
  *out = nullptr;
  if (!config_ok(cfg)) return CKV_E_INVALID;
  if (!device_arena || ((uintptr_t)device_arena % kAlign) != 0 || arena_bytes < layout_of(cfg).total)
    return CKV_E_ARENA;
  ckv_cache* c = new (std::nothrow) ckv_cache(*cfg, false, (char*)device_arena, arena_bytes);
  if (!c) return CKV_E_INVALID;
  *out = c;
  return CKV_OK;
}

ckv_status ckv_cache_create_dry(const ckv_config* cfg, ckv_cache** out) {
  if (!out) return CKV_E_INVALID;
  *out = nullptr;
  if (!config_ok(cfg)) return CKV_E_INVALID;
  ckv_cache* c = new (std::nothrow) ckv_cache(*cfg, true, nullptr, 0);
  if (!c) return CKV_E_INVALID;
  *out = c;
  return CKV_OK;
}

ckv_status ckv_cache_reset(ckv_cache* c) {
  if (!c) return CKV_E_INVALID;
  c->sched.reset();
  for (int& n : c->text_len) n = 0;
  return CKV_OK;
}

ckv_status ckv_cache_destroy(ckv_cache* c) {
  if (!c) return CKV_E_INVALID;
  delete c;
  return CKV_OK;
}

ckv_status ckv_rope_append(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q, const void* k,
                           const void* v, void* q_rot, void* stream) {
  return append_impl(c, layer, step, chunk, q, k, v, q_rot, stream, QkNorm());
}

ckv_status ckv_sink_build(ckv_cache* c, int32_t layer, const void* q, const void* k, const void* v, void* q_rot,
                          void* stream) {
  return sink_impl(c, layer, q, k, v, q_rot, stream, QkNorm());
}

ckv_status ckv_norm_rope_append(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q,
                                const void* k, const void* v, const float* q_gain, const float* k_gain, float eps,
                                void* q_rot, void* stream) {
  QkNorm n;
  n.q_gain = q_gain;
  n.k_gain = k_gain;
  n.eps = eps;
  if (!norm_ok(n)) return CKV_E_INVALID;
  return append_impl(c, layer, step, chunk, q, k, v, q_rot, stream, n);
}

ckv_status ckv_norm_sink_build(ckv_cache* c, int32_t layer, const void* q, const void* k, const void* v,
                               const float* q_gain, const float* k_gain, float eps, void* q_rot, void* stream) {
  QkNorm n;
  n.q_gain = q_gain;
  n.k_gain = k_gain;
  n.eps = eps;
  if (!norm_ok(n)) return CKV_E_INVALID;
  return sink_impl(c, layer, q, k, v, q_rot, stream, n);
}

ckv_status ckv_chunk_attention(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q_rot,
                               void* out, void* stream) {
  return attention_impl(c, layer, step, chunk, q_rot, out, stream, false);
}

ckv_status ckv_chunk_attention_static(ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, const void* q_rot,
                                      void* out, void* stream) {
  return attention_impl(c, layer, step, chunk, q_rot, out, stream, true);
}

ckv_status ckv_text_store(ckv_cache* c, int32_t layer, const void* k_text, const void* v_text, int32_t n_text,
                          void* stream) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(k_text) || !ptr_ok(v_text)) return CKV_E_INVALID;
  if (layer < 0 || layer >= c->cfg.num_layers || n_text < 1 || n_text > CKV_MAX_TEXT_TOKENS) return CKV_E_INVALID;
  if (!c->dry) {
    hipStream_t s = (hipStream_t)stream;
    ckv_status st = ensure_device(c, s);
    if (st != CKV_OK) return st;
    ckv::TextStoreParams p;
    p.k = (const bf16_t*)k_text;
    p.v = (const bf16_t*)v_text;
    p.k_dst = c->text_k(layer);
    p.vt_dst = c->text_vt(layer);
    p.n_text = n_text;
    p.max_text = CKV_MAX_TEXT_TOKENS;
    p.num_heads = c->cfg.num_heads;
    if (ckv::launch_text_store(p, c->cfg.head_dim, s) != hipSuccess) return CKV_E_HIP;
  }
  c->text_len[layer] = n_text;
  return CKV_OK;
}

ckv_status ckv_cross_attention(ckv_cache* c, int32_t layer, int32_t chunk, const void* q, void* out, void* stream) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(q) || !ptr_ok(out)) return CKV_E_INVALID;
  if (layer < 0 || layer >= c->cfg.num_layers || chunk < 0 || chunk >= c->cfg.max_chunks) return CKV_E_INVALID;
  const int n_text = c->text_len[layer];
  if (n_text == 0) return CKV_E_STATE;
  if (c->dry) return CKV_OK;
  hipStream_t s = (hipStream_t)stream;
  ckv_status st = ensure_device(c, s);
  if (st != CKV_OK) return st;
  const long long d = c->cfg.head_dim;
  ckv::AttnParams p;
  std::memset(&p, 0, sizeof(p));
  for (int i = 0; i < 3; ++i) {  // one run: the stored context
    p.k[i] = c->text_k(layer);
    p.vt[i] = c->text_vt(layer);
    p.k_head_stride[i] = (long long)CKV_MAX_TEXT_TOKENS * d;
    p.vt_head_stride[i] = d * CKV_MAX_TEXT_TOKENS;
    p.vt_row_stride[i] = CKV_MAX_TEXT_TOKENS;
    p.seg_end[i] = n_text;
  }
  p.q = (const bf16_t*)q;
  p.out = (bf16_t*)out;
  p.n_queries = c->tokens(chunk);
  p.n_keys = n_text;
  p.num_heads = c->cfg.num_heads;
  p.n_splits = splits_for(c->num_cus, c->cfg.num_heads, p.n_queries, p.n_keys);
  p.q_tiles = (p.n_queries + ckv::kAttnQueryTile - 1) / ckv::kAttnQueryTile;
  p.key_tiles = (p.n_keys + ckv::kAttnKeyTile - 1) / ckv::kAttnKeyTile;
  p.scale_log2 = c->scale() * 1.4426950408889634f;
  p.part_o = (uint16_t*)(c->arena + c->L.part_o_off);
  p.part_lse = (float*)(c->arena + c->L.part_lse_off);
  return ckv::launch_chunk_attention(p, c->cfg.head_dim, s) == hipSuccess ? CKV_OK : CKV_E_HIP;
}

ckv_status ckv_window(const ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, ckv_segment* segs,
                      int32_t max_segs, int32_t* n_segs) {
  if (!c || !segs || !n_segs) return CKV_E_INVALID;
  if (layer < 0 || layer >= c->cfg.num_layers || chunk < 0 || chunk >= c->cfg.max_chunks) return CKV_E_INVALID;
  if (!((step >= 0 && step < c->cfg.num_steps) || (chunk == 0 && step == CKV_STEP_SINK))) return CKV_E_INVALID;
  ckv::Segment tmp[3];
  const int n = c->sched.window(chunk, tmp);
  if (n > max_segs) return CKV_E_INVALID;
  for (int i = 0; i < n; ++i) {
    segs[i].kind = tmp[i].kind;
    segs[i].first_slot = tmp[i].first_slot;
    segs[i].chunk_first = tmp[i].chunk_first;
    segs[i].n_chunks = tmp[i].n_chunks;
    segs[i].n_tokens = tmp[i].n_tokens;
  }
  *n_segs = n;
  return CKV_OK;
}

ckv_status ckv_ring_slot(const ckv_cache* c, int32_t chunk, int32_t* slot) {
  if (!c || !slot || chunk < 1 || chunk >= c->cfg.max_chunks) return CKV_E_INVALID;
  *slot = c->sched.slot_of(chunk);
  return CKV_OK;
}

ckv_status ckv_debug_copy_kv(const ckv_cache* c, int32_t layer, int32_t step, int32_t chunk, void* k_out,
                             void* v_out, void* stream) {
  if (!c) return CKV_E_INVALID;
  if (!ptr_ok(k_out) || !ptr_ok(v_out)) return CKV_E_INVALID;
  ckv_status st = to_status(c->sched.check_live(layer, step, chunk));
  if (st != CKV_OK) return st;
  if (c->dry) return CKV_OK;
  const long long d = c->cfg.head_dim;
  ckv::CopyKVParams p;
  if (chunk == 0) {
    p.k_src = c->sink_k(layer);
    p.vt_src = c->sink_vt(layer);
    p.k_head_stride = (long long)c->L.n0 * d;
    p.vt_head_stride = d * c->L.n0;
    p.vt_row_stride = c->L.n0;
  } else {
    const int slot = c->sched.slot_of(chunk);
    p.k_src = c->ring_k(layer, step) + (size_t)slot * c->L.n1 * d;
    p.vt_src = c->ring_vt(layer, step) + (size_t)slot * c->L.n1;
    p.k_head_stride = (long long)c->L.ring_rows * d;
    p.vt_head_stride = d * c->L.ring_rows;
    p.vt_row_stride = c->L.ring_rows;
  }
  p.n_tokens = c->tokens(chunk);
  p.num_heads = c->cfg.num_heads;
  p.k_out = (bf16_t*)k_out;
  p.v_out = (bf16_t*)v_out;
  return ckv::launch_copy_kv(p, c->cfg.head_dim, (hipStream_t)stream) == hipSuccess ? CKV_OK : CKV_E_HIP;
}

int32_t ckv_attention_splits(const ckv_cache* c, int32_t n_queries, int32_t n_keys) {
  if (!c || n_queries <= 0 || n_keys <= 0) return 0;
  return splits_for(c->num_cus, c->cfg.num_heads, n_queries, n_keys);
}

const char* ckv_status_string(ckv_status st) {
  switch (st) {
    case CKV_OK: return "ok";
    case CKV_E_INVALID: return "invalid argument";
    case CKV_E_ORDER: return "call out of schedule order";
    case CKV_E_STATE: return "cache state does not allow this call";
    case CKV_E_ARENA: return "arena too small, null or misaligned";
    case CKV_E_HIP: return "HIP launch or runtime failure";
  }
  return "unknown status";
}

}  // extern "C"
