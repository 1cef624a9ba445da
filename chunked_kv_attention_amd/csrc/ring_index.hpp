// Host-side schedule state and ring indexer for same-step chunk attention.
//
// Window rule ("PhysisServe -- Wan2.2 5B" model card, "Inference profile"):
// chunk c >= 1 at step s reads the sink, the step-s K/V of the most recent
// min(c-1, W) chunks among 1..c-1, and its own K/V.  Every (layer, step) keeps
// the noisy K/V of chunks >= 1 in a ring of R = W + 1 chunk slots: chunk c
// sits in slot (c-1) mod R.  Because a chunk's append comes before its
// attention, R = W + 1 lets the append evict exactly chunk c-W-1, the one
// chunk c no longer reads, while chunks c-W .. c stay live; their slots are
// contiguous modulo R, so the window is the sink plus at most two runs of
// slots.
#pragma once

#include <cstdint>
#include <vector>

namespace ckv {

struct Segment {
  int32_t kind;         // 0 = sink area, 1 = run of ring slots
  int32_t first_slot;   // -1 for the sink area
  int32_t chunk_first;  // chunk id of the run's first chunk
  int32_t n_chunks;
  int32_t n_tokens;
};

enum class Check { kOk, kInvalid, kOrder, kState };

// Who last wrote a layer's sink area.
enum : int32_t { kAreaEmpty = -2, kAreaSink = -1 };  // >= 0: chunk 0's step

class Schedule {
 public:
  Schedule(int32_t layers, int32_t steps, int32_t window, int32_t max_chunks, int32_t first_tokens,
           int32_t chunk_tokens)
      : layers_(layers), steps_(steps), window_(window), max_chunks_(max_chunks),
        first_tokens_(first_tokens), chunk_tokens_(chunk_tokens) {
    reset();
  }

  void reset() {
    next_.assign(static_cast<size_t>(layers_) * steps_, 1);
    area_.assign(layers_, kAreaEmpty);
  }

  int32_t ring_slots() const { return window_ + 1; }
  int32_t slot_of(int32_t chunk) const { return (chunk - 1) % ring_slots(); }

  // Validation of one call against the state; no state change.
  Check check_append(int32_t layer, int32_t step, int32_t chunk) const {
    if (!valid_layer(layer) || step < 0 || step >= steps_ || chunk < 0 || chunk >= max_chunks_)
      return Check::kInvalid;
    if (chunk == 0) return area_[layer] == kAreaSink ? Check::kState : Check::kOk;
    if (area_[layer] != kAreaSink) return Check::kState;
    return next_[idx(layer, step)] == chunk ? Check::kOk : Check::kOrder;
  }
  Check check_sink_build(int32_t layer) const {
    if (!valid_layer(layer)) return Check::kInvalid;
    return area_[layer] == kAreaSink ? Check::kState : Check::kOk;
  }
  Check check_attention(int32_t layer, int32_t step, int32_t chunk) const {
    if (!valid_layer(layer) || chunk < 0 || chunk >= max_chunks_) return Check::kInvalid;
    if (chunk == 0) {
      if (step == kAreaSink) return area_[layer] == kAreaSink ? Check::kOk : Check::kState;
      if (step < 0 || step >= steps_) return Check::kInvalid;
      return area_[layer] == step ? Check::kOk : Check::kState;
    }
    if (step < 0 || step >= steps_) return Check::kInvalid;
    if (area_[layer] != kAreaSink) return Check::kState;
    return next_[idx(layer, step)] == chunk + 1 ? Check::kOk : Check::kOrder;
  }
  // A stored chunk that can still be read back.
  Check check_live(int32_t layer, int32_t step, int32_t chunk) const {
    if (!valid_layer(layer) || chunk < 0 || chunk >= max_chunks_) return Check::kInvalid;
    if (chunk == 0) {
      if (step == kAreaSink) return area_[layer] == kAreaSink ? Check::kOk : Check::kState;
      if (step < 0 || step >= steps_) return Check::kInvalid;
      return area_[layer] == step ? Check::kOk : Check::kState;
    }
    if (step < 0 || step >= steps_) return Check::kInvalid;
    const int32_t newest = next_[idx(layer, step)] - 1;
    if (area_[layer] != kAreaSink || chunk > newest || chunk < newest - window_) return Check::kState;
    return Check::kOk;
  }

  // State transitions (call only after the matching check returned kOk and the
  // launch succeeded).
  void commit_append(int32_t layer, int32_t step, int32_t chunk) {
    if (chunk == 0)
      area_[layer] = step;
    else
      next_[idx(layer, step)] = chunk + 1;
  }
  void commit_sink_build(int32_t layer) { area_[layer] = kAreaSink; }

  // Window of (step, chunk) as <= 3 segments in key order.  Config-only.
  int32_t window(int32_t chunk, Segment* out) const {
    if (chunk == 0) {
      out[0] = Segment{0, -1, 0, 1, first_tokens_};
      return 1;
    }
    int32_t n = 0;
    out[n++] = Segment{0, -1, 0, 1, first_tokens_};
    const int32_t lo = chunk - window_ > 1 ? chunk - window_ : 1;  // oldest noisy chunk read
    int32_t count = chunk - lo + 1;                                 // window chunks + self
    int32_t first = lo;
    int32_t slot = slot_of(lo);
    while (count > 0) {
      const int32_t run = (ring_slots() - slot) < count ? (ring_slots() - slot) : count;
      out[n++] = Segment{1, slot, first, run, run * chunk_tokens_};
      count -= run;
      first += run;
      slot = 0;
    }
    return n;
  }

 private:
  bool valid_layer(int32_t l) const { return l >= 0 && l < layers_; }
  size_t idx(int32_t l, int32_t s) const { return static_cast<size_t>(l) * steps_ + s; }

  int32_t layers_, steps_, window_, max_chunks_, first_tokens_, chunk_tokens_;
  std::vector<int32_t> next_;  // per (layer, step): next chunk >= 1 expected
  std::vector<int32_t> area_;  // per layer: who last wrote the sink area
};

}  // namespace ckv
