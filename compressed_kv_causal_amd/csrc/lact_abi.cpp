// lact_abi.cpp -- the extern "C" boundary of liblact.so (declared in include/lact.h):
// argument and state checks, the cache buffer layout, host bookkeeping, kernel launches.
// Every check runs before anything is enqueued; a failed call leaves the state unchanged.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "lact.h"
#include "plan.hpp"

namespace {

thread_local std::string g_last_error;

lact_status fail(lact_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_bytes(int32_t dt) { return dt == LACT_F32 ? 4 : (dt == LACT_BF16 ? 2 : 1); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

lact_status check_cfg(const lact_cfg* c) {
  if (!c) return fail(LACT_E_INVALID, "cfg is NULL");
  if (c->heads < 1 || c->grid_h < 1 || c->grid_w < 1)
    return fail(LACT_E_SHAPE, "heads, grid_h and grid_w must be >= 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(LACT_E_SHAPE, "head_dim must be 64 or 128");
  if (c->window_frames < 0 || c->mem_slots < 0)
    return fail(LACT_E_SHAPE, "window_frames and mem_slots must be >= 0");
  if (c->ratio < 1 || c->ratio > 16) return fail(LACT_E_SHAPE, "ratio must be in 1..16");
  if (c->max_block_frames < 1) return fail(LACT_E_SHAPE, "max_block_frames must be >= 1");
  if (c->ref_frames < 0) return fail(LACT_E_SHAPE, "ref_frames must be >= 0");
  const int64_t kf = (int64_t)c->ref_frames + c->mem_slots + c->window_frames + c->max_block_frames;
  if (kf > LACT_MAX_KEY_FRAMES)
    return fail(LACT_E_CAPACITY, "ref_frames + mem_slots + window_frames + max_block_frames exceeds " +
                                     std::to_string(LACT_MAX_KEY_FRAMES));
  const int64_t T = (int64_t)c->grid_h * c->grid_w;
  if (T > LACT_MAX_TOKENS)
    return fail(LACT_E_CAPACITY, "grid_h * grid_w exceeds " + std::to_string(LACT_MAX_TOKENS));
  if (T * c->heads * c->head_dim > (int64_t(1) << 28) || kf * T > (int64_t(1) << 24))
    return fail(LACT_E_CAPACITY, "frame or key length too large");
  const bool ok_dt = (c->q_dtype == LACT_F32 && c->kv_dtype == LACT_F32) ||
                     (c->q_dtype == LACT_BF16 &&
                      (c->kv_dtype == LACT_BF16 || c->kv_dtype == LACT_FP8_E4M3));
  if (!ok_dt)
    return fail(LACT_E_DTYPE, "supported (q, kv) dtypes: (F32, F32), (BF16, BF16), (BF16, FP8_E4M3)");
  if (c->rope_mode == 3) {
    for (int i = 0; i < 3; ++i)
      if (c->rope_split[i] < 2 || (c->rope_split[i] & 1))
        return fail(LACT_E_SHAPE, "rope_split parts must be even and >= 2");
    if (c->rope_split[0] + c->rope_split[1] + c->rope_split[2] != c->head_dim)
      return fail(LACT_E_SHAPE, "rope_split must sum to head_dim");
  } else if (c->rope_mode != 1) {
    return fail(LACT_E_SHAPE, "rope_mode must be 1 or 3");
  }
  if (!(c->rope_theta > 1.0f) || !std::isfinite(c->rope_theta))
    return fail(LACT_E_INVALID, "rope_theta must be finite and > 1");
  return LACT_OK;
}

int64_t rope_table_entries(const lact_cfg& c) {
  const int64_t kf = (int64_t)c.ref_frames + c.mem_slots + c.window_frames + c.max_block_frames;
  const int64_t T = (int64_t)c.grid_h * c.grid_w;
  if (c.rope_mode == 1) return kf * T * (c.head_dim / 2);
  return kf * (c.rope_split[0] / 2) + (int64_t)c.grid_h * (c.rope_split[1] / 2) +
         (int64_t)c.grid_w * (c.rope_split[2] / 2);
}

lact_status check_members(int32_t n) {
  if (n < 1 || n > LACT_MAX_MEMBERS)
    return fail(LACT_E_CAPACITY, "n_members " + std::to_string(n) + " outside 1.." +
                                     std::to_string(LACT_MAX_MEMBERS));
  return LACT_OK;
}

// Persistent regions of member 0 first (member m's at + m * member_bytes), then the
// staging shared by all members.
void compute_layout(const lact_cfg& c, int32_t members, lact_layout* L) {
  std::memset(L, 0, sizeof(*L));
  const int64_t T = (int64_t)c.grid_h * c.grid_w;
  const int64_t fe = T * c.heads * c.head_dim;  // elements per frame
  const size_t kvb = elem_bytes(c.kv_dtype);
  const int32_t R = c.window_frames + c.max_block_frames + c.ratio - 1;
  const int32_t KF = c.ref_frames + c.mem_slots + c.window_frames + c.max_block_frames;
  const int32_t B = c.max_block_frames, M = c.mem_slots;
  const bool fp8 = c.kv_dtype == LACT_FP8_E4M3;
  const size_t fb = (size_t)fe * kvb;
  const size_t ob = (size_t)fe * elem_bytes(c.q_dtype);  // one frame in the operand dtype
  const size_t sb = (size_t)T * c.heads * 4;  // one frame of f32 row scales
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L->ring_k = take(fb * R);
  L->ring_v = take(fb * R);
  L->mem_k = take(fb * M);
  L->mem_v = take(fb * M);
  L->ref_k = take(fb * (size_t)c.ref_frames);
  L->ref_v = take(fb * (size_t)c.ref_frames);
  if (fp8) {
    L->ring_k_scale = take(sb * R);
    L->ring_v_scale = take(sb * R);
    L->mem_k_scale = take(sb * M);
    L->mem_v_scale = take(sb * M);
    L->ref_k_scale = take(sb * (size_t)c.ref_frames);
    L->ref_v_scale = take(sb * (size_t)c.ref_frames);
  }
  L->member_bytes = off;
  L->members = members;
  off = L->member_bytes * (size_t)members;
  L->krot = take(ob * KF);
  L->qrot = take(ob * B);
  L->vcur = take(fb * B);
  L->vcur_scale = take(fp8 ? sb * B : 0);
  L->vscale = take(fp8 ? 3 * sizeof(float) * (size_t)c.heads * ((size_t)KF * (size_t)T + lact::kVscalePad) : 0);
  L->rope_table = take(sizeof(float) * 2 * (size_t)rope_table_entries(c));
  L->attn_flags = take(sizeof(int32_t) * (size_t)c.heads * (size_t)((B * T + 255) / 256));
  L->vmax = take(fp8 ? sizeof(float) * lact::kVmaxParts * (size_t)c.heads : 0);
  L->total = off;
  L->frame_bytes = fb;
  L->ring_slots = R;
  L->key_frames_max = KF;
}

}  // namespace

struct lact_cache {
  lact_cfg cfg;
  lact_layout lay;
  lact::Planner plan;
  char* buf;
  bool table_ready = false;
  bool staged = false;        // the staging holds staged_member's operands ...
  uint64_t staged_version = 0;  // ... of this state version
  int32_t staged_frames = 0;
  int32_t staged_member = 0;
  const void* staged_v = nullptr;  // the block's V as passed to the RoPE call (bf16, f32)
  bool hist_built = false;    // the staged history (krot, FP8 vscale) is hist_member's ...
  uint64_t hist_version = 0;  // ... at this version
  int32_t hist_member = 0;
  std::vector<uint8_t> ref_valid;  // per member: the reference segment has been stored
  lact_cache(const lact_cfg& c, const lact_layout& l, void* b)
      : cfg(c), lay(l), plan(c), buf(static_cast<char*>(b)), ref_valid((size_t)l.members, 0) {}

  int32_t T() const { return cfg.grid_h * cfg.grid_w; }
  int32_t members() const { return lay.members; }
  // shared staging regions
  void* at(size_t off) const { return buf + off; }
  // member m's persistent regions
  void* mat(int32_t m, size_t off) const { return buf + (size_t)m * lay.member_bytes + off; }
  float* fat(int32_t m, size_t off) const {
    return cfg.kv_dtype == LACT_FP8_E4M3 ? reinterpret_cast<float*>(mat(m, off)) : nullptr;
  }
  bool all_refs() const {
    for (uint8_t v : ref_valid)
      if (!v) return false;
    return true;
  }
  lact::HistMap hist() const {
    lact::HistMap m;
    m.ref_len = cfg.ref_frames;
    m.mem_len = plan.mem_len();
    m.win_len = plan.win_len();
    m.M = cfg.mem_slots;
    m.R = plan.ring_slots();
    m.mem_slot0 = cfg.mem_slots > 0 ? (int32_t)(plan.first_mem_group() % cfg.mem_slots) : 0;
    m.ring_slot0 = (int32_t)(plan.evicted() % plan.ring_slots());
    return m;
  }
};

struct lact_plan {
  lact::Planner p;
  explicit lact_plan(const lact_cfg& c) : p(c) {}
};

static lact_status hip_fail(hipError_t e, const char* what) {
  return fail(LACT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

extern "C" {

const char* lact_last_error(void) { return g_last_error.c_str(); }

lact_status lact_set_footprint(const lact_cfg* cfg, int32_t n_members, size_t* device_bytes) {
  lact_status st = check_cfg(cfg);
  if (st == LACT_OK) st = check_members(n_members);
  if (st != LACT_OK) return st;
  if (!device_bytes) return fail(LACT_E_INVALID, "device_bytes is NULL");
  lact_layout L;
  compute_layout(*cfg, n_members, &L);
  *device_bytes = L.total;
  return LACT_OK;
}

lact_status lact_cache_footprint(const lact_cfg* cfg, size_t* device_bytes) {
  return lact_set_footprint(cfg, 1, device_bytes);
}

lact_status lact_set_layout(const lact_cfg* cfg, int32_t n_members, lact_layout* out) {
  lact_status st = check_cfg(cfg);
  if (st == LACT_OK) st = check_members(n_members);
  if (st != LACT_OK) return st;
  if (!out) return fail(LACT_E_INVALID, "out is NULL");
  compute_layout(*cfg, n_members, out);
  return LACT_OK;
}

lact_status lact_cache_layout(const lact_cfg* cfg, lact_layout* out) {
  return lact_set_layout(cfg, 1, out);
}

lact_status lact_set_init(const lact_cfg* cfg, int32_t n_members, void* device_buf, size_t bytes,
                          lact_cache** out) {
  lact_status st = check_cfg(cfg);
  if (st == LACT_OK) st = check_members(n_members);
  if (st != LACT_OK) return st;
  if (!out) return fail(LACT_E_INVALID, "out is NULL");
  if (!device_buf || !aligned(device_buf, 256))
    return fail(LACT_E_INVALID, "device_buf must be non-NULL and 256-byte aligned");
  lact_layout L;
  compute_layout(*cfg, n_members, &L);
  if (bytes < L.total)
    return fail(LACT_E_CAPACITY, "device buffer of " + std::to_string(bytes) + " bytes; need " +
                                     std::to_string(L.total));
  lact_cache* c = nullptr;
  try {  // the handle's per-member table allocates too; no exception crosses the C ABI
    c = new lact_cache(*cfg, L, device_buf);
  } catch (const std::bad_alloc&) {
    return fail(LACT_E_CAPACITY, "host allocation of the handle failed");
  }
  *out = c;
  return LACT_OK;
}

lact_status lact_cache_init(const lact_cfg* cfg, void* device_buf, size_t bytes, lact_cache** out) {
  return lact_set_init(cfg, 1, device_buf, bytes, out);
}

lact_status lact_cache_destroy(lact_cache* cache) {
  delete cache;
  return LACT_OK;
}

lact_status lact_member_rope_reset_apply(lact_cache* c, int32_t member, const void* q,
                                         const void* k_cur, const void* v_cur, int32_t n_frames,
                                         void* stream) {
  if (!c) return fail(LACT_E_INVALID, "cache is NULL");
  if (member < 0 || member >= c->members())
    return fail(LACT_E_INVALID, "member " + std::to_string(member) + " outside 0.." +
                                    std::to_string(c->members() - 1));
  if (!q || !k_cur || !v_cur || !aligned(q, 16) || !aligned(k_cur, 16) || !aligned(v_cur, 16))
    return fail(LACT_E_INVALID, "q, k_cur, v_cur must be non-NULL and 16-byte aligned");
  if (n_frames < 1 || n_frames > c->cfg.max_block_frames)
    return fail(LACT_E_CAPACITY, "n_frames " + std::to_string(n_frames) + " outside 1.." +
                                     std::to_string(c->cfg.max_block_frames));
  if (c->cfg.ref_frames > 0 && !c->ref_valid[(size_t)member])
    return fail(LACT_E_STATE, "the reference segment has not been set (lact_ref_set)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const lact_cfg& g = c->cfg;
  // Under stream capture the launches run only when the graph does: the table and the
  // history are then recorded into the graph every time (each replay is self-contained),
  // and neither is marked as present for later eager calls.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess) cap = hipStreamCaptureStatusNone;
  const bool capturing = cap != hipStreamCaptureStatusNone;
  if (!c->table_ready || capturing) {
    lact::RopeTableArgs t;
    t.table = static_cast<float2*>(c->at(c->lay.rope_table));
    t.rope_mode = g.rope_mode;
    t.split_t = g.rope_split[0];
    t.split_h = g.rope_split[1];
    t.split_w = g.rope_split[2];
    t.D = g.head_dim;
    t.T = c->T();
    t.grid_h = g.grid_h;
    t.grid_w = g.grid_w;
    t.key_frames_max = c->lay.key_frames_max;
    t.theta = (double)g.rope_theta;
    t.entries = rope_table_entries(g);
    hipError_t e = lact::launch_rope_table(t, s);
    if (e != hipSuccess) return hip_fail(e, "rope table launch");
    if (!capturing) c->table_ready = true;
  }
  lact::RopeArgs a;
  a.q = q;
  a.k_cur = k_cur;
  a.v_cur = v_cur;
  const int32_t m = member;
  a.ring_k = c->mat(m, c->lay.ring_k);
  a.mem_k = c->mat(m, c->lay.mem_k);
  a.ring_v = c->mat(m, c->lay.ring_v);
  a.mem_v = c->mat(m, c->lay.mem_v);
  a.ref_k = c->mat(m, c->lay.ref_k);
  a.ref_v = c->mat(m, c->lay.ref_v);
  a.ring_k_scale = c->fat(m, c->lay.ring_k_scale);
  a.mem_k_scale = c->fat(m, c->lay.mem_k_scale);
  a.ring_v_scale = c->fat(m, c->lay.ring_v_scale);
  a.mem_v_scale = c->fat(m, c->lay.mem_v_scale);
  a.ref_k_scale = c->fat(m, c->lay.ref_k_scale);
  a.ref_v_scale = c->fat(m, c->lay.ref_v_scale);
  a.krot = c->at(c->lay.krot);
  a.qrot = c->at(c->lay.qrot);
  a.vcur = c->at(c->lay.vcur);
  const bool fp8 = g.kv_dtype == LACT_FP8_E4M3;
  a.vcur_scale = fp8 ? reinterpret_cast<float*>(c->at(c->lay.vcur_scale)) : nullptr;
  a.table = static_cast<const float2*>(c->at(c->lay.rope_table));
  a.hist = c->hist();
  const bool rebuild = capturing || !(c->hist_built && c->hist_version == c->plan.version() &&
                                       c->hist_member == member);
  a.hist_rows = rebuild ? 1 : 0;
  a.n_cur = n_frames;
  a.T = c->T();
  a.H = g.heads;
  a.D = g.head_dim;
  a.grid_h = g.grid_h;
  a.grid_w = g.grid_w;
  a.key_frames_max = c->lay.key_frames_max;
  a.block_frames_max = g.max_block_frames;
  a.rope_mode = g.rope_mode;
  a.split_t = g.rope_split[0];
  a.split_h = g.rope_split[1];
  a.split_w = g.rope_split[2];
  a.in_dtype = g.q_dtype;
  a.kv_dtype = g.kv_dtype;
  a.q_scale = (float)(1.4426950408889634 / std::sqrt((double)g.head_dim));
  hipError_t e = lact::launch_rope(a, s);
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  if (fp8) {
    lact::VscaleArgs v;
    v.ring_v_scale = a.ring_v_scale;
    v.mem_v_scale = a.mem_v_scale;
    v.ref_v_scale = a.ref_v_scale;
    v.vcur_scale = a.vcur_scale;
    v.vscale = reinterpret_cast<float*>(c->at(c->lay.vscale));
    v.vmax = reinterpret_cast<float*>(c->at(c->lay.vmax));
    v.hist = a.hist;
    v.T = c->T();
    v.H = g.heads;
    v.Lk = (c->plan.history_frames() + n_frames) * c->T();
    v.key_frames_max = c->lay.key_frames_max;
    e = lact::launch_vscale_stage(v, s);
    if (e != hipSuccess) return hip_fail(e, "V scale staging launch");
  }
  c->hist_built = !capturing;
  c->hist_version = c->plan.version();
  c->hist_member = member;
  c->staged = true;
  c->staged_version = c->plan.version();
  c->staged_frames = n_frames;
  c->staged_member = member;
  c->staged_v = v_cur;
  return LACT_OK;
}

static lact_status refuse_set(const lact_cache* c, const char* call) {
  return fail(LACT_E_INVALID, std::string("the handle is a set of ") + std::to_string(c->members()) +
                                  " members: name one with lact_member_" + call);
}

lact_status lact_rope_reset_apply(lact_cache* c, const void* q, const void* k_cur, const void* v_cur,
                                  int32_t n_frames, void* stream) {
  if (c && c->members() > 1) return refuse_set(c, "rope_reset_apply");
  return lact_member_rope_reset_apply(c, 0, q, k_cur, v_cur, n_frames, stream);
}

}  // extern "C"

// ---- the exact pass's work queue in a library-held array ---------------------------------
// For lact_member_block_attention_static: one int32 per (head, 256-row query tile), in a
// file-scope device array instead of the cache buffer's attn_flags region.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device, with that device current, and kept.
static __device__ __align__(256) int32_t scratch[LACT_STATIC_QUEUE_MAX];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that runs `stream` (the current device for
// the null stream).
lact_status scratch_address(hipStream_t stream, int32_t** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LACT_E_CAPACITY, "device index " + std::to_string(dev) + " outside 0.." +
                                     std::to_string(kMaxDevices - 1));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return LACT_OK;
}
}  // namespace

// Block attention of `member`; `static_queue` takes the exact pass's work queue from
// `scratch` instead of the cache buffer.
static lact_status block_attention_impl(lact_cache* c, int32_t member, const int32_t* q_block_frames,
                                        int32_t n_q_blocks, void* out, float* lse, void* stream,
                                        bool static_queue) {
  if (!c) return fail(LACT_E_INVALID, "cache is NULL");
  if (member < 0 || member >= c->members())
    return fail(LACT_E_INVALID, "member " + std::to_string(member) + " outside 0.." +
                                    std::to_string(c->members() - 1));
  if (!out || !aligned(out, 16)) return fail(LACT_E_INVALID, "out must be non-NULL and 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(LACT_E_INVALID, "lse must be 4-byte aligned");
  if (!c->staged || c->staged_version != c->plan.version())
    return fail(LACT_E_STATE, "lact_rope_reset_apply has not run at the present state");
  if (c->staged_member != member)
    return fail(LACT_E_STATE, "the staging holds member " + std::to_string(c->staged_member) +
                                  ", not member " + std::to_string(member));
  const lact_cfg& g = c->cfg;
  const int32_t T = c->T();
  lact::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  if (q_block_frames == nullptr) {
    a.n_blocks = 1;
    a.block_end[0] = c->staged_frames * T;
  } else {
    if (n_q_blocks < 1 || n_q_blocks > LACT_MAX_Q_BLOCKS)
      return fail(LACT_E_CAPACITY, "n_q_blocks outside 1.." + std::to_string(LACT_MAX_Q_BLOCKS));
    int32_t sum = 0;
    for (int32_t b = 0; b < n_q_blocks; ++b) {
      if (q_block_frames[b] < 1) return fail(LACT_E_SHAPE, "every query block needs >= 1 frame");
      sum += q_block_frames[b];
      a.block_end[b] = sum * T;
    }
    if (sum != c->staged_frames)
      return fail(LACT_E_SHAPE, "q_block_frames sum to " + std::to_string(sum) + ", staged " +
                                    std::to_string(c->staged_frames));
    a.n_blocks = n_q_blocks;
  }
  a.q = c->at(c->lay.qrot);
  a.k = c->at(c->lay.krot);
  // the block's V: an FP8 cache's as staged e4m3 codes, otherwise where the caller passed
  // it to the RoPE call (same layout and dtype as the staging; see lact.h)
  a.v_cur = g.kv_dtype == LACT_FP8_E4M3 ? static_cast<const void*>(c->at(c->lay.vcur)) : c->staged_v;
  a.out = out;
  a.lse = lse;
  if (static_queue) {
    const int64_t items = (int64_t)g.heads * ((c->staged_frames * (int64_t)T + 255) / 256);
    if (items > LACT_STATIC_QUEUE_MAX)
      return fail(LACT_E_CAPACITY, "heads x 256-row query tiles = " + std::to_string(items) +
                                       " exceeds LACT_STATIC_QUEUE_MAX (" +
                                       std::to_string(LACT_STATIC_QUEUE_MAX) + ")");
    lact_status st = scratch_address(static_cast<hipStream_t>(stream), &a.flags);
    if (st != LACT_OK) return st;
  } else {
    a.flags = reinterpret_cast<int32_t*>(c->at(c->lay.attn_flags));
  }
  a.q_head_stride = (int64_t)g.max_block_frames * T * g.head_dim;
  a.k_head_stride = (int64_t)c->lay.key_frames_max * T * g.head_dim;
  a.hist = c->hist();
  // V is read where it is stored: the member's reference, memory and ring rows, and the
  // staged block (an FP8 cache's as e4m3 codes, with every key's row scale in vscale)
  a.v_ring = c->mat(member, c->lay.ring_v);
  a.v_mem = c->mat(member, c->lay.mem_v);
  a.v_ref = c->mat(member, c->lay.ref_v);
  if (g.kv_dtype == LACT_FP8_E4M3) {
    a.v_fp8 = 1;
    a.vscale = reinterpret_cast<const float*>(c->at(c->lay.vscale));
    a.vmax = reinterpret_cast<const float*>(c->at(c->lay.vmax));
    a.vs_head_stride = (int64_t)c->lay.key_frames_max * T + lact::kVscalePad;
    a.vs_plane = a.vs_head_stride * g.heads;
  }
  a.T = T;
  a.H = g.heads;
  a.D = g.head_dim;
  a.Lq = c->staged_frames * T;
  a.Lhist = c->plan.history_frames() * T;
  a.Lk = a.Lhist + a.Lq;
  hipError_t e = lact::launch_attention(a, g.q_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return LACT_OK;
}

extern "C" {

lact_status lact_member_block_attention(lact_cache* c, int32_t member, const int32_t* q_block_frames,
                                        int32_t n_q_blocks, void* out, float* lse, void* stream) {
  return block_attention_impl(c, member, q_block_frames, n_q_blocks, out, lse, stream, false);
}

lact_status lact_member_block_attention_static(lact_cache* c, int32_t member,
                                               const int32_t* q_block_frames, int32_t n_q_blocks,
                                               void* out, float* lse, void* stream) {
  return block_attention_impl(c, member, q_block_frames, n_q_blocks, out, lse, stream, true);
}

lact_status lact_block_attention(lact_cache* c, const int32_t* q_block_frames, int32_t n_q_blocks,
                                 void* out, float* lse, void* stream) {
  if (c && c->members() > 1) return refuse_set(c, "block_attention");
  return lact_member_block_attention(c, 0, q_block_frames, n_q_blocks, out, lse, stream);
}

lact_status lact_member_ref_set(lact_cache* c, int32_t member, const void* k_ref, const void* v_ref,
                                int32_t n_frames, void* stream) {
  if (!c) return fail(LACT_E_INVALID, "cache is NULL");
  if (member < 0 || member >= c->members())
    return fail(LACT_E_INVALID, "member " + std::to_string(member) + " outside 0.." +
                                    std::to_string(c->members() - 1));
  if (!k_ref || !v_ref || !aligned(k_ref, 16) || !aligned(v_ref, 16))
    return fail(LACT_E_INVALID, "k_ref and v_ref must be non-NULL and 16-byte aligned");
  const lact_cfg& g = c->cfg;
  if (g.ref_frames < 1) return fail(LACT_E_STATE, "this cache has no reference segment (ref_frames = 0)");
  if (n_frames != g.ref_frames)
    return fail(LACT_E_SHAPE, "n_frames " + std::to_string(n_frames) + " != ref_frames " +
                                  std::to_string(g.ref_frames));
  lact::RingWriteArgs a;
  a.src[0] = k_ref;
  a.src[1] = v_ref;
  a.ring[0] = c->mat(member, c->lay.ref_k);
  a.ring[1] = c->mat(member, c->lay.ref_v);
  a.ring_scale[0] = c->fat(member, c->lay.ref_k_scale);
  a.ring_scale[1] = c->fat(member, c->lay.ref_v_scale);
  a.members = 1;
  a.src_mstride = 0;
  a.ring_mstride = 0;
  a.slot0 = 0;
  a.n_frames = n_frames;
  a.R = n_frames;
  a.T = c->T();
  a.H = g.heads;
  a.D = g.head_dim;
  a.in_dtype = g.q_dtype;
  a.kv_dtype = g.kv_dtype;
  hipError_t e = lact::launch_ring_write(a, (int64_t)n_frames * a.T * a.H, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "reference write launch");
  c->ref_valid[(size_t)member] = 1;
  if (c->hist_member == member) c->hist_built = false;  // its rotated reference keys (and
  if (c->staged_member == member) c->staged = false;    // FP8 values) are restaged
  return LACT_OK;
}

lact_status lact_ref_set(lact_cache* c, const void* k_ref, const void* v_ref, int32_t n_frames,
                         void* stream) {
  if (c && c->members() > 1) return refuse_set(c, "ref_set");
  return lact_member_ref_set(c, 0, k_ref, v_ref, n_frames, stream);
}

lact_status lact_kv_ring_append(lact_cache* c, const void* k_new, const void* v_new, int32_t n_frames,
                                void* stream) {
  if (!c) return fail(LACT_E_INVALID, "cache is NULL");
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
    return fail(LACT_E_INVALID, "k_new and v_new must be non-NULL and 16-byte aligned");
  std::string why = c->plan.check_append(n_frames);
  if (!why.empty())
    return fail(n_frames < 1 || n_frames > c->plan.max_block() ? LACT_E_CAPACITY : LACT_E_STATE, why);
  const lact_cfg& g = c->cfg;
  lact::RingWriteArgs a;
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.ring[0] = c->mat(0, c->lay.ring_k);
  a.ring[1] = c->mat(0, c->lay.ring_v);
  a.ring_scale[0] = c->fat(0, c->lay.ring_k_scale);
  a.ring_scale[1] = c->fat(0, c->lay.ring_v_scale);
  a.members = c->members();
  a.src_mstride = (int64_t)n_frames * c->T() * g.heads * g.head_dim * (int64_t)elem_bytes(g.q_dtype);
  a.ring_mstride = (int64_t)c->lay.member_bytes;
  a.slot0 = c->plan.raw_slot(c->plan.frames_appended());
  a.n_frames = n_frames;
  a.R = c->plan.ring_slots();
  a.T = c->T();
  a.H = g.heads;
  a.D = g.head_dim;
  a.in_dtype = g.q_dtype;
  a.kv_dtype = g.kv_dtype;
  hipError_t e = lact::launch_ring_write(a, (int64_t)n_frames * a.T * a.H, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  c->plan.append(n_frames);
  return LACT_OK;
}

lact_status lact_convkv_compress(lact_cache* c, const float* w_k, const float* b_k, const float* w_v,
                                 const float* b_v, void* stream, int32_t* slots_written) {
  if (!c) return fail(LACT_E_INVALID, "cache is NULL");
  if (!w_k || !b_k || !w_v || !b_v || !aligned(w_k, 16) || !aligned(b_k, 16) || !aligned(w_v, 16) ||
      !aligned(b_v, 16))
    return fail(LACT_E_INVALID, "weights and biases must be non-NULL and 16-byte aligned");
  const lact_cfg& g = c->cfg;
  const int32_t ready = c->plan.ready_groups();
  const int32_t M = g.mem_slots;
  const int32_t written = ready < M ? ready : M;
  const int64_t G = c->plan.groups_compressed();
  const int64_t first = G + ready - written;  // earlier groups would be overwritten at once
  lact::CompressArgs a;
  std::memset(&a, 0, sizeof(a));
  a.ring[0] = c->mat(0, c->lay.ring_k);
  a.ring[1] = c->mat(0, c->lay.ring_v);
  a.ring_scale[0] = c->fat(0, c->lay.ring_k_scale);
  a.ring_scale[1] = c->fat(0, c->lay.ring_v_scale);
  a.mem[0] = c->mat(0, c->lay.mem_k);
  a.mem[1] = c->mat(0, c->lay.mem_v);
  a.mem_scale[0] = c->fat(0, c->lay.mem_k_scale);
  a.mem_scale[1] = c->fat(0, c->lay.mem_v_scale);
  a.members = c->members();
  a.mstride = (int64_t)c->lay.member_bytes;
  a.w_mstride = (int64_t)g.heads * g.head_dim * g.ratio;
  a.b_mstride = (int64_t)g.heads * g.head_dim;
  a.w[0] = w_k;
  a.w[1] = w_v;
  a.b[0] = b_k;
  a.b[1] = b_v;
  a.r = g.ratio;
  a.R = c->plan.ring_slots();
  a.T = c->T();
  a.H = g.heads;
  a.D = g.head_dim;
  a.kv_dtype = g.kv_dtype;
  for (int32_t done = 0; done < written;) {
    const int32_t n = written - done < lact::kMaxGroupsPerLaunch ? written - done : lact::kMaxGroupsPerLaunch;
    for (int32_t i = 0; i < n; ++i) {
      const int64_t grp = first + done + i;
      a.in_slot0[i] = (int32_t)((grp * g.ratio) % a.R);
      a.out_slot[i] = (int32_t)(grp % M);
    }
    a.n_groups = n;
    hipError_t e = lact::launch_compress(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "compress launch");
    done += n;
  }
  c->plan.consume_groups(ready);
  if (slots_written) *slots_written = written;
  return LACT_OK;
}

lact_status lact_cache_state(const lact_cache* c, lact_state* out) {
  if (!c || !out) return fail(LACT_E_INVALID, "cache and out must be non-NULL");
  c->plan.state(out);
  out->staged_frames = c->staged ? c->staged_frames : 0;
  out->staged_valid = (c->staged && c->staged_version == c->plan.version()) ? 1 : 0;
  out->ref_valid = c->all_refs() ? 1 : 0;
  out->staged_member = c->staged_member;
  return LACT_OK;
}

lact_status lact_cache_keys(const lact_cache* c, int32_t n_cur, lact_key_frame* out, int32_t cap,
                            int32_t* n_out) {
  if (!c || !n_out) return fail(LACT_E_INVALID, "cache and n_out must be non-NULL");
  if (n_cur < 0 || n_cur > c->cfg.max_block_frames) return fail(LACT_E_CAPACITY, "n_cur out of range");
  if (cap < 0 || (cap > 0 && !out)) return fail(LACT_E_INVALID, "bad out/cap");
  *n_out = c->plan.key_frames(n_cur, out, cap);
  return LACT_OK;
}

lact_status lact_plan_create(const lact_cfg* cfg, lact_plan** out) {
  lact_status st = check_cfg(cfg);
  if (st != LACT_OK) return st;
  if (!out) return fail(LACT_E_INVALID, "out is NULL");
  lact_plan* p = new (std::nothrow) lact_plan(*cfg);
  if (!p) return fail(LACT_E_CAPACITY, "host allocation failed");
  *out = p;
  return LACT_OK;
}

lact_status lact_plan_destroy(lact_plan* p) {
  delete p;
  return LACT_OK;
}

lact_status lact_plan_append(lact_plan* p, int32_t n_frames) {
  if (!p) return fail(LACT_E_INVALID, "plan is NULL");
  std::string why = p->p.check_append(n_frames);
  if (!why.empty())
    return fail(n_frames < 1 || n_frames > p->p.max_block() ? LACT_E_CAPACITY : LACT_E_STATE, why);
  p->p.append(n_frames);
  return LACT_OK;
}

lact_status lact_plan_compress(lact_plan* p, int64_t* groups, int32_t cap, int32_t* n_groups,
                               int32_t* n_written) {
  if (!p || !n_groups) return fail(LACT_E_INVALID, "plan and n_groups must be non-NULL");
  if (cap < 0 || (cap > 0 && !groups)) return fail(LACT_E_INVALID, "bad groups/cap");
  const int32_t ready = p->p.ready_groups();
  const int64_t G = p->p.groups_compressed();
  for (int32_t i = 0; i < ready && i < cap; ++i) groups[i] = G + i;
  *n_groups = ready;
  if (n_written) *n_written = ready < p->p.mem_slots() ? ready : p->p.mem_slots();
  p->p.consume_groups(ready);
  return LACT_OK;
}

lact_status lact_plan_state(const lact_plan* p, lact_state* out) {
  if (!p || !out) return fail(LACT_E_INVALID, "plan and out must be non-NULL");
  p->p.state(out);
  return LACT_OK;
}

lact_status lact_plan_keys(const lact_plan* p, int32_t n_cur, lact_key_frame* out, int32_t cap,
                           int32_t* n_out) {
  if (!p || !n_out) return fail(LACT_E_INVALID, "plan and n_out must be non-NULL");
  if (n_cur < 0) return fail(LACT_E_CAPACITY, "n_cur out of range");
  if (cap < 0 || (cap > 0 && !out)) return fail(LACT_E_INVALID, "bad out/cap");
  *n_out = p->p.key_frames(n_cur, out, cap);
  return LACT_OK;
}

}  // extern "C"
