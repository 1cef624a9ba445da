// C-ABI of the streaming causal 3D convolution (declared in
// include/ckv_conv.h).
//
// Host responsibilities: validate the config and every call, lay out the
// caller's arena ([packed weights | float32 bias | 2-frame cache | zero
// row | split partials]), keep the stream position (frames consumed since
// the last reset), plan which tiles split their reduction by time offset, and
// launch the kernels on the caller's stream.  The cache needs no clearing
// on reset: a frame before the video is never read from it (the kernel takes
// the zero row instead).  Nothing here allocates device memory or
// synchronises.
#include "ckv_conv.h"

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <new>

#include "kernels.hpp"

namespace {

using ckv::bf16_t;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool config_ok(const ckv_conv_config* c) {
  if (!c) return false;
  if (c->height < 1 || c->width < 1 || c->max_frames < 1) return false;
  if (c->in_channels < 64 || c->in_channels % 64 != 0) return false;
  if (c->out_channels < ckv::kConvChannelTile || c->out_channels % ckv::kConvChannelTile != 0) return false;
  if (c->kt < 1 || c->kt > CKV_CONV_CACHE_T + 1) return false;
  if ((c->kh != 1 && c->kh != 3) || (c->kw != 1 && c->kw != 3)) return false;
  // 32-bit lane offsets into the packed weights of one tap and pixel indexes
  const long long taps = (long long)c->kt * c->kh * c->kw;
  if ((long long)c->out_channels * c->in_channels * 2 >= (1LL << 31)) return false;
  if (taps * c->out_channels * c->in_channels * 2 >= (1LL << 40)) return false;
  if ((long long)c->max_frames * c->height * c->width >= (1LL << 31) - ckv::kConvPixelTile) return false;
  return true;
}

struct ConvLayout {
  size_t w_off = 0, w_bytes = 0;
  size_t bias_off = 0, cache_off = 0, frame_bytes = 0, zero_off = 0, part_off = 0, total = 0;
};

ConvLayout layout_of(const ckv_conv_config& c) {
  ConvLayout L;
  const size_t taps = (size_t)c.kt * c.kh * c.kw;
  L.w_off = 0;
  L.w_bytes = taps * c.out_channels * c.in_channels * sizeof(bf16_t);
  L.bias_off = align_up(L.w_off + L.w_bytes);
  L.cache_off = align_up(L.bias_off + sizeof(float) * c.out_channels);
  L.frame_bytes = (size_t)c.height * c.width * c.in_channels * sizeof(bf16_t);
  L.zero_off = align_up(L.cache_off + CKV_CONV_CACHE_T * L.frame_bytes);
  L.part_off = align_up(L.zero_off + sizeof(bf16_t) * c.in_channels);
  // float32 partials of up to kt splits of the largest chunk (none for kt = 1)
  const size_t part = c.kt > 1 ? sizeof(float) * c.kt * (size_t)c.max_frames * c.height * c.width * c.out_channels : 0;
  L.total = align_up(L.part_off + part);
  return L;
}

// How a call's units (pixel tile, channel tile) run, with two workgroups per
// CU as the slots: all of them split kt ways by time offset when even the
// split parts fill at most two rounds of slots; otherwise whole, except a
// last, partly filled round, whose units are split when their parts fit in
// one round; whole throughout for kt = 1.
struct SplitPlan {
  int whole;   // units run over all taps
  int splits;  // parts of every later unit
};

SplitPlan plan_for(const ckv_conv_config& c, int frames, int num_cus) {
  const long long pix = (long long)frames * c.height * c.width;
  const long long units = (pix + ckv::kConvPixelTile - 1) / ckv::kConvPixelTile * (c.out_channels / ckv::kConvChannelTile);
  const long long slots = 2LL * (num_cus > 0 ? num_cus : 256);
  if (c.kt == 1) return SplitPlan{(int)units, 1};
  if (units * c.kt <= 2 * slots) return SplitPlan{0, c.kt};
  const long long tail = units % slots;
  if (tail > 0 && tail * c.kt <= slots) return SplitPlan{(int)(units - tail), c.kt};
  return SplitPlan{(int)units, 1};
}

bool ptr_ok(const void* p) { return p != nullptr && ((uintptr_t)p % 16) == 0; }

}  // namespace

struct ckv_conv {
  ckv_conv_config cfg;
  ConvLayout L;
  char* arena;  // null for a dry state
  bool dry;
  bool weights_set;
  long long position;  // frames consumed since the last reset
  int num_cus;         // of the device the first call ran on (256 for a dry state)
  ckv_conv(const ckv_conv_config& c, char* a, bool d)
      : cfg(c), L(layout_of(c)), arena(a), dry(d), weights_set(false), position(0), num_cus(d ? 256 : 0) {}
};

namespace {
ckv_status ensure_cus(ckv_conv* c) {
  if (c->num_cus == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CKV_E_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return CKV_E_HIP;
    c->num_cus = cus > 0 ? cus : 256;
  }
  return CKV_OK;
}
}  // namespace

extern "C" {

size_t ckv_conv_bytes(const ckv_conv_config* cfg) { return config_ok(cfg) ? layout_of(*cfg).total : 0; }

ckv_status ckv_conv_create(const ckv_conv_config* cfg, void* device_arena, size_t arena_bytes, ckv_conv** out) {
  if (!out) return CKV_E_INVALID;
  *out = nullptr;
  if (!config_ok(cfg)) return CKV_E_INVALID;
  if (!device_arena || (uintptr_t)device_arena % kAlign != 0 || arena_bytes < layout_of(*cfg).total)
    return CKV_E_ARENA;
  *out = new (std::nothrow) ckv_conv(*cfg, static_cast<char*>(device_arena), false);
  return *out ? CKV_OK : CKV_E_INVALID;
}

ckv_status ckv_conv_create_dry(const ckv_conv_config* cfg, ckv_conv** out) {
  if (!out) return CKV_E_INVALID;
  *out = nullptr;
  if (!config_ok(cfg)) return CKV_E_INVALID;
  *out = new (std::nothrow) ckv_conv(*cfg, nullptr, true);
  return *out ? CKV_OK : CKV_E_INVALID;
}

ckv_status ckv_conv_set_weights(ckv_conv* c, const void* weight, const void* bias, void* stream) {
  if (!c || !ptr_ok(weight) || (bias && (uintptr_t)bias % 2 != 0)) return CKV_E_INVALID;
  if (!c->dry) {
    ckv::ConvPackParams p{};
    p.weight = static_cast<const bf16_t*>(weight);
    p.bias = static_cast<const bf16_t*>(bias);
    p.w_packed = reinterpret_cast<bf16_t*>(c->arena + c->L.w_off);
    p.bias_out = reinterpret_cast<float*>(c->arena + c->L.bias_off);
    p.zero = reinterpret_cast<bf16_t*>(c->arena + c->L.zero_off);
    p.c_out = c->cfg.out_channels;
    p.c_in = c->cfg.in_channels;
    p.taps = c->cfg.kt * c->cfg.kh * c->cfg.kw;
    p.zero_u4 = c->cfg.in_channels / 8;
    if (ckv::launch_conv_pack(p, static_cast<hipStream_t>(stream)) != hipSuccess) return CKV_E_HIP;
  }
  c->weights_set = true;
  return CKV_OK;
}

ckv_status ckv_conv_reset(ckv_conv* c) {
  if (!c) return CKV_E_INVALID;
  c->position = 0;
  return CKV_OK;
}

ckv_status ckv_causal_conv(ckv_conv* c, const void* x, int32_t frames, void* y, void* stream) {
  if (!c || !ptr_ok(x) || !ptr_ok(y)) return CKV_E_INVALID;
  if (frames < 1 || frames > c->cfg.max_frames) return CKV_E_INVALID;
  const size_t pix = (size_t)frames * c->cfg.height * c->cfg.width;
  const uintptr_t x0 = (uintptr_t)x, x1 = x0 + pix * c->cfg.in_channels * sizeof(bf16_t);
  const uintptr_t y0 = (uintptr_t)y, y1 = y0 + pix * c->cfg.out_channels * sizeof(bf16_t);
  if (x0 < y1 && y0 < x1) return CKV_E_INVALID;  // the kernel reads x while it writes y
  if (!c->weights_set) return CKV_E_STATE;
  if (!c->dry) {
    if (ensure_cus(c) != CKV_OK) return CKV_E_HIP;
    ckv::ConvParams p{};
    p.x = static_cast<const bf16_t*>(x);
    p.y = static_cast<bf16_t*>(y);
    p.w = reinterpret_cast<const bf16_t*>(c->arena + c->L.w_off);
    p.bias = reinterpret_cast<const float*>(c->arena + c->L.bias_off);
    p.cache = reinterpret_cast<bf16_t*>(c->arena + c->L.cache_off);
    p.zero = reinterpret_cast<const bf16_t*>(c->arena + c->L.zero_off);
    p.k0 = c->position;
    p.frames = frames;
    p.height = c->cfg.height;
    p.width = c->cfg.width;
    p.c_in = c->cfg.in_channels;
    p.c_out = c->cfg.out_channels;
    p.kt = c->cfg.kt;
    p.kh = c->cfg.kh;
    p.kw = c->cfg.kw;
    p.m_tiles = (int)((pix + ckv::kConvPixelTile - 1) / ckv::kConvPixelTile);
    const SplitPlan plan = plan_for(c->cfg, frames, c->num_cus);
    p.whole = plan.whole;
    p.splits = plan.splits;
    p.part = reinterpret_cast<float*>(c->arena + c->L.part_off);
    if (ckv::launch_causal_conv(p, static_cast<hipStream_t>(stream)) != hipSuccess) return CKV_E_HIP;
  }
  c->position += frames;
  return CKV_OK;
}

int64_t ckv_conv_position(const ckv_conv* c) { return c ? c->position : -1; }

int32_t ckv_conv_splits(const ckv_conv* c, int32_t frames, int32_t* whole_units) {
  if (!c || frames < 1 || frames > c->cfg.max_frames) return 0;
  const SplitPlan plan = plan_for(c->cfg, frames, c->num_cus);
  if (whole_units) *whole_units = plan.whole;
  return plan.splits;
}

ckv_status ckv_conv_destroy(ckv_conv* c) {
  if (!c) return CKV_E_INVALID;
  delete c;
  return CKV_OK;
}

}  // extern "C"
