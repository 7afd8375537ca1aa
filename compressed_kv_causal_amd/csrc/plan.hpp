// plan.hpp -- host bookkeeping of one ConvKV cache: counters, eviction, pending groups,
// memory ring and the key-frame table.  Plain C++ (no HIP), so it runs and is tested
// anywhere.
//
// The memory it manages (SoulX-LiveAct pages): an exact recent window plus a long-term
// memory built by a 1D convolution at a fixed 5:1 ratio into a fixed length (news
// summary "SoulX-LiveAct - Soul App ...", technical principle, ConvKV Memory bullet; press
// release digi.china.com, technical-principle paragraph), with append-only reuse of
// cached KV and compression once between blocks (walkthrough "SoulX-LiveAct", sections
// "ConvKV Memory" and "Streaming Pipeline").
//
// Key frames in attention order: [reference (fixed, ref_frames frames) | memory | window |
// current]; the temporal position of a key frame is its rank.
//
// Counters: F frames appended, G groups compressed, E = max(0, F - W) evicted.  Group g =
// frames [r*g, r*g + r) -> memory slot g mod M.  Up to r-1 evicted frames wait (pending)
// for their group and are not attended.  Raw slot of frame f = f mod R, R = W + B_max + r - 1,
// which can never hold two live frames: live = pending (< r) + window (<= W) + new (<= B_max).
#pragma once

#include <cstdint>
#include <string>

#include "lact.h"

namespace lact {

class Planner {
 public:
  explicit Planner(const lact_cfg& cfg)
      : ref_(cfg.ref_frames), W_(cfg.window_frames), M_(cfg.mem_slots), r_(cfg.ratio),
        B_(cfg.max_block_frames) {
    R_ = W_ + B_ + r_ - 1;
  }

  int64_t frames_appended() const { return F_; }
  int64_t groups_compressed() const { return G_; }
  int64_t evicted() const { return F_ > W_ ? F_ - W_ : 0; }
  int32_t pending() const { return static_cast<int32_t>(evicted() - static_cast<int64_t>(r_) * G_); }
  int32_t win_len() const { return static_cast<int32_t>(F_ - evicted()); }
  int32_t mem_len() const { return G_ < M_ ? static_cast<int32_t>(G_) : M_; }
  int32_t ring_slots() const { return R_; }
  int32_t mem_slots() const { return M_; }
  int32_t max_block() const { return B_; }
  uint64_t version() const { return version_; }
  // oldest group present in memory and oldest frame of the window
  int64_t first_mem_group() const { return G_ - mem_len(); }
  int32_t ref_frames() const { return ref_; }
  // key frames before the current block: [reference | memory | window]
  int32_t history_frames() const { return ref_ + mem_len() + win_len(); }

  int32_t raw_slot(int64_t frame) const { return static_cast<int32_t>(frame % R_); }
  int32_t mem_slot(int64_t group) const { return M_ > 0 ? static_cast<int32_t>(group % M_) : -1; }

  // Checks of an append of n frames; empty string if allowed.
  std::string check_append(int32_t n) const;
  void append(int32_t n) {
    F_ += n;
    ++version_;
  }

  // Complete groups waiting to be compressed.
  int32_t ready_groups() const {
    return static_cast<int32_t>((evicted() - static_cast<int64_t>(r_) * G_) / r_);
  }
  void consume_groups(int32_t n) {
    if (n > 0) {
      G_ += n;
      ++version_;
    }
  }

  // Key-frame table in attention order for a block of n_cur frames; returns the count.
  int32_t key_frames(int32_t n_cur, lact_key_frame* out, int32_t cap) const;
  void state(lact_state* st) const;

 private:
  int32_t ref_, W_, M_, r_, B_, R_;
  int64_t F_ = 0, G_ = 0;
  uint64_t version_ = 0;
};

}  // namespace lact
