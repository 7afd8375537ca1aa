// Drives the host planner (compressed_kv_causal_amd/csrc/plan.cpp) over long schedules of
// several configurations (with a reference segment, window-only, memory-only, uneven
// blocks), for a build with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_sanitizers.py).  Checks the counters against their closed form after every
// append and compress, and fills key tables into exactly sized and undersized buffers.
#include <cstdio>
#include <cstring>
#include <vector>

#include "plan.hpp"

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::fprintf(stderr, "line %d: %s\n", __LINE__, #c);        \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static lact_cfg cfg(int W, int M, int r, int B, int ref) {
  lact_cfg c;
  std::memset(&c, 0, sizeof(c));
  c.heads = 2;
  c.head_dim = 64;
  c.grid_h = 2;
  c.grid_w = 2;
  c.window_frames = W;
  c.mem_slots = M;
  c.ratio = r;
  c.max_block_frames = B;
  c.ref_frames = ref;
  return c;
}

int main() {
  const int configs[][5] = {{8, 16, 5, 8, 0}, {8, 16, 5, 8, 2}, {4, 0, 5, 2, 0},
                            {0, 10, 5, 3, 1}, {6, 16, 5, 8, 0}, {3, 4, 3, 7, 2}};
  for (const auto& k : configs) {
    const lact_cfg c = cfg(k[0], k[1], k[2], k[3], k[4]);
    lact::Planner p(c);
    int64_t F = 0;
    for (int step = 0; step < 1000; ++step) {
      const int n = 1 + (step * 7) % k[3];
      CHECK(p.check_append(n).empty());
      CHECK(!p.check_append(0).empty() && !p.check_append(k[3] + 1).empty());
      const int32_t count = p.key_frames(n, nullptr, 0);
      std::vector<lact_key_frame> keys(static_cast<size_t>(count));
      CHECK(p.key_frames(n, keys.data(), count) == count);
      std::vector<lact_key_frame> few(2);
      CHECK(p.key_frames(n, few.data(), 2) == count);
      for (int32_t i = 0; i < count; ++i) CHECK(keys[static_cast<size_t>(i)].t_pos == i);
      p.append(n);
      F += n;
      p.consume_groups(p.ready_groups());
      lact_state st;
      p.state(&st);
      const int64_t E = F > k[0] ? F - k[0] : 0;
      CHECK(st.F == F && st.E == E && st.G == E / k[2] && st.pending == E % k[2]);
      CHECK(st.mem_len == (st.G < k[1] ? st.G : k[1]));
      CHECK(p.history_frames() == k[4] + st.mem_len + st.win_len);
    }
  }
  if (fails) std::fprintf(stderr, "%d checks failed\n", fails);
  return fails ? 1 : 0;
}
