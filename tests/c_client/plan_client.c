/* A plain C client of liblact: built by tests/test_host_abi.py with gcc against
 * include/lact.h, it checks the structs and calls as a C compiler sees them (the Python
 * binding mirrors them by hand).  Host-only calls: sizing, layout, the planner, errors.
 * The planner's counters are checked against the schedule's closed form after every step
 * of 1000: F = n B, E = max(0, F - W), G = floor(E / r) (every complete group consumed),
 * pending = E mod r, mem_len = min(G, M), win_len = min(W, F), and the key table
 * [memory oldest..newest | window | current] with t = rank.  Exit status 0 = all held. */
#include <stdio.h>
#include <string.h>

#include "lact.h"

static int fails = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "line %d: %s\n", __LINE__, #cond);             \
      ++fails;                                                       \
    }                                                                \
  } while (0)

static lact_cfg cfg_512(void) {
  lact_cfg c;
  memset(&c, 0, sizeof(c));
  c.heads = 40;
  c.head_dim = 128;
  c.grid_h = 32;
  c.grid_w = 32;
  c.window_frames = 8;
  c.mem_slots = 16;
  c.ratio = 5;
  c.max_block_frames = 8;
  c.kv_dtype = LACT_BF16;
  c.q_dtype = LACT_BF16;
  c.rope_mode = 3;
  c.rope_split[0] = 44;
  c.rope_split[1] = 42;
  c.rope_split[2] = 42;
  c.rope_theta = 10000.0f;
  c.ref_frames = 0;
  return c;
}

int main(void) {
  lact_cfg c = cfg_512();
  const int64_t W = 8, M = 16, r = 5, B = 8, R = W + B + r - 1;

  /* sizing and layout */
  size_t bytes = 0;
  lact_layout L;
  CHECK(lact_cache_footprint(&c, &bytes) == LACT_OK);
  CHECK(lact_cache_layout(&c, &L) == LACT_OK);
  CHECK(bytes > 0 && L.total == bytes);
  CHECK(L.ring_slots == R && L.key_frames_max == M + W + B);
  CHECK(L.frame_bytes == (size_t)1024 * 40 * 128 * 2);
  CHECK(L.ring_k % 256 == 0 && L.mem_k % 256 == 0 && L.krot % 256 == 0 && L.total % 256 == 0);
  CHECK(L.ring_v >= L.ring_k + R * L.frame_bytes && L.mem_k >= L.ring_v + R * L.frame_bytes);
  CHECK(L.members == 1 && L.member_bytes <= L.krot);

  /* errors: refused with a status and a message, nothing created */
  lact_cfg bad = c;
  bad.head_dim = 96;
  lact_plan* none = NULL;
  CHECK(lact_plan_create(&bad, &none) == LACT_E_SHAPE && none == NULL);
  CHECK(strlen(lact_last_error()) > 0);

  /* the planner over 1000 steps of B frames */
  lact_plan* p = NULL;
  CHECK(lact_plan_create(&c, &p) == LACT_OK && p != NULL);
  if (!p) return 1;
  CHECK(lact_plan_append(p, 0) == LACT_E_CAPACITY);
  CHECK(lact_plan_append(p, (int32_t)B + 1) == LACT_E_CAPACITY);
  lact_key_frame keys[LACT_MAX_KEY_FRAMES];
  int64_t groups[64];
  for (int64_t n = 1; n <= 1000; ++n) {
    int32_t ng = -1, nw = -1;
    CHECK(lact_plan_append(p, (int32_t)B) == LACT_OK);
    CHECK(lact_plan_compress(p, groups, 64, &ng, &nw) == LACT_OK);
    lact_state s;
    CHECK(lact_plan_state(p, &s) == LACT_OK);
    const int64_t F = n * B, E = F > W ? F - W : 0, G = E / r;
    const int64_t mem = G < M ? G : M, win = W < F ? W : F;
    CHECK(s.F == F && s.E == E && s.G == G && s.pending == (int32_t)(E % r));
    CHECK(s.mem_len == (int32_t)mem && s.win_len == (int32_t)win && s.ring_slots == (int32_t)R);
    CHECK(nw == (ng < M ? ng : M));
    for (int32_t i = 0; i < ng; ++i) CHECK(groups[i] == G - ng + i);
    int32_t nk = -1;
    CHECK(lact_plan_keys(p, (int32_t)B, keys, LACT_MAX_KEY_FRAMES, &nk) == LACT_OK);
    CHECK(nk == (int32_t)(mem + win + B));
    for (int32_t i = 0; i < nk && i < LACT_MAX_KEY_FRAMES; ++i) {
      CHECK(keys[i].t_pos == i);
      if (i < mem) {
        const int64_t g = G - mem + i;
        CHECK(keys[i].segment == LACT_SEG_MEMORY && keys[i].absolute_id == g &&
              keys[i].physical_slot == (int32_t)(g % M));
      } else if (i < mem + win) {
        const int64_t f = F - win + (i - mem);
        CHECK(keys[i].segment == LACT_SEG_WINDOW && keys[i].absolute_id == f &&
              keys[i].physical_slot == (int32_t)(f % R));
      } else {
        CHECK(keys[i].segment == LACT_SEG_CURRENT && keys[i].physical_slot == (int32_t)(i - mem - win));
      }
    }
    if (fails) break;
  }
  CHECK(lact_plan_destroy(p) == LACT_OK);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("c client: sizing, layout, errors and 1000 planner steps hold\n");
  return fails ? 1 : 0;
}
