// plan.cpp -- see plan.hpp.
#include "plan.hpp"

namespace lact {

std::string Planner::check_append(int32_t n) const {
  if (n < 1 || n > B_)
    return "append of " + std::to_string(n) + " frames; allowed 1.." + std::to_string(B_);
  if (pending() >= r_)
    return "a complete group of evicted frames is waiting: call lact_convkv_compress first";
  return std::string();
}

int32_t Planner::key_frames(int32_t n_cur, lact_key_frame* out, int32_t cap) const {
  int32_t rank = 0;
  auto put = [&](int32_t seg, int32_t slot, int64_t id) {
    if (out && rank < cap) {
      out[rank].segment = seg;
      out[rank].physical_slot = slot;
      out[rank].absolute_id = id;
      out[rank].t_pos = rank;
      out[rank].reserved = 0;
    }
    ++rank;
  };
  for (int32_t i = 0; i < ref_; ++i) put(LACT_SEG_REF, i, i);
  for (int64_t g = first_mem_group(); g < G_; ++g) put(LACT_SEG_MEMORY, mem_slot(g), g);
  for (int64_t f = evicted(); f < F_; ++f) put(LACT_SEG_WINDOW, raw_slot(f), f);
  for (int32_t i = 0; i < n_cur; ++i) put(LACT_SEG_CURRENT, i, F_ + i);
  return rank;
}

void Planner::state(lact_state* st) const {
  st->F = F_;
  st->E = evicted();
  st->G = G_;
  st->win_len = win_len();
  st->mem_len = mem_len();
  st->pending = pending();
  st->ring_slots = R_;
  st->version = version_;
  st->staged_frames = 0;
  st->staged_valid = 0;
  st->ref_valid = 0;
  st->staged_member = 0;
}

}  // namespace lact
