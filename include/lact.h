/*
 * lact.h -- C ABI of liblact.so: ConvKV-memory block-causal attention on MI355X (gfx950).
 *
 * One AR step of one self-attention layer at one diffusion step, as the SoulX-LiveAct pages
 * describe it:
 *   - the KV of already generated latent frames is kept append-only and reused, only the new
 *     block's KV is added (walkthrough "SoulX-LiveAct", sections "ConvKV Memory" and
 *     "Streaming Pipeline");
 *   - a recent window of exact KV frames is kept; older frames are compressed by a
 *     lightweight 1D convolution at a fixed 5:1 ratio into a fixed-length long-term memory
 *     (news summary "SoulX-LiveAct - Soul App ...", section "technical principle", ConvKV
 *     Memory bullet; press release digi.china.com, technical-principle paragraph; arXiv
 *     listing 2603.11746, Figure 3 caption);
 *   - RoPE positions are reset so they stay bounded (press release, technical-principle
 *     paragraph; news summary, ConvKV Memory bullet);
 *   - the current block's queries attend over [reference | memory | window | current]
 *     under the block-wise causal mask of block size m (walkthrough, section "Neighbor
 *     Forcing"; the reference image's KV is the first of the context's partitions);
 *   - the footprint is constant for any video length (walkthrough, "Streaming Pipeline").
 *
 * Step order per AR step and per cache (one cache per layer and diffusion step):
 *   lact_rope_reset_apply -> lact_block_attention -> lact_kv_ring_append -> lact_convkv_compress
 * Compression runs once between blocks (walkthrough, "Streaming Pipeline").
 *
 * Conventions for every call below:
 *   - Tensor pointers are HIP device pointers owned by the caller, 16-byte aligned, each
 *     holding at least the extent its call states (the library cannot see buffer sizes and
 *     reads or writes exactly those extents).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). All device work is
 *     enqueued asynchronously on it; no call synchronises with the device and no call
 *     allocates device memory.
 *   - Every check runs before anything is enqueued. On error the call returns a non-OK
 *     status, the cache state is unchanged and lact_last_error() holds a message.
 *   - A cache handle is not thread-safe; separate handles are independent.  Successive
 *     calls on one handle depend on each other's device work (the staging, the ring and
 *     the memory): issue them on one stream, or order the streams with events.
 *   - A handle holds one cache (lact_cache_init) or a set of n_members caches of one cfg
 *     (lact_set_init: one per layer and diffusion step) that advance together: they share
 *     the bookkeeping, the staging area and the RoPE table, and append and compress run for
 *     all members in one launch each.
 *   - Layouts are token-major: a frame is T = grid_h*grid_w tokens, row-major over the
 *     (h, w) patch grid; per token H heads of D channels; channel c = h*D + d.
 */
#ifndef LACT_H
#define LACT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LACT_OK = 0,
  LACT_E_INVALID = 1,  /* null or misaligned pointer, bad argument                      */
  LACT_E_SHAPE = 2,    /* unsupported or inconsistent sizes                              */
  LACT_E_CAPACITY = 3, /* too many frames / blocks / key frames, buffer too small        */
  LACT_E_DTYPE = 4,    /* unsupported dtype combination                                  */
  LACT_E_STATE = 5,    /* call out of order (see each call)                              */
  LACT_E_HIP = 6       /* a HIP launch or runtime call failed                            */
} lact_status;

typedef enum { LACT_F32 = 0, LACT_BF16 = 1, LACT_FP8_E4M3 = 2 } lact_dtype;

/* Fixed at init. Symbols: H heads, D head_dim, T = grid_h*grid_w tokens per latent frame,
 * W window frames, M memory slots, r compression ratio (= conv kernel = stride),
 * B_max the largest block appended or attended in one call. */
typedef struct {
  int32_t heads, head_dim, grid_h, grid_w;
  int32_t window_frames, mem_slots, ratio, max_block_frames;
  int32_t kv_dtype;      /* lact_dtype: F32, BF16 or FP8_E4M3 (e4m3 codes + per-(token,head) f32 scale) */
  int32_t q_dtype;       /* lact_dtype of q, k_cur, v_cur, k_new, v_new and out: F32 or BF16.
                            F32 requires kv F32; BF16 requires kv BF16 or FP8_E4M3.       */
  int32_t rope_mode;     /* 1: 1D, position p = t*T + u over all D channels;
                            3: 3D, (t, h, w) over the channel split rope_split            */
  int32_t rope_split[3]; /* 3D: d_t, d_h, d_w, each even, sum = head_dim                  */
  float rope_theta;      /* RoPE base, e.g. 10000                                         */
  int32_t ref_frames;    /* reference segment: frames of a fixed KV prefix (the reference
                            image's part of the context) attended before the memory by
                            every step; 0 = none.  Set once with lact_ref_set.           */
} lact_cfg;

/* Supported: head_dim 64 or 128; heads >= 1; 1 <= T <= LACT_MAX_TOKENS; W >= 0; M >= 0;
 * 1 <= r <= 16; 1 <= B_max; ref_frames >= 0; ref_frames + M + W + B_max <=
 * LACT_MAX_KEY_FRAMES; T * heads * head_dim <= 2^28 and (ref_frames + M + W + B_max) * T
 * <= 2^24 (LACT_E_CAPACITY otherwise).  LACT_MAX_TOKENS keeps every launch grid within
 * the device's per-dimension limits. */
#define LACT_MAX_TOKENS 262144
#define LACT_MAX_KEY_FRAMES 256
#define LACT_MAX_Q_BLOCKS 16
#define LACT_MAX_MEMBERS 1024

/* Segment of a key frame in attention order. */
enum { LACT_SEG_MEMORY = 0, LACT_SEG_WINDOW = 1, LACT_SEG_CURRENT = 2, LACT_SEG_REF = 3 };

/* One key frame in attention order
 * [reference | memory oldest..newest | window oldest..newest | current]. */
typedef struct {
  int32_t segment;       /* LACT_SEG_*                                                    */
  int32_t physical_slot; /* reference: index i; memory: g mod M; window: f mod R;
                            current: index in the block                                   */
  int64_t absolute_id;   /* reference: i; memory: group g; window and current: frame f     */
  int32_t t_pos;         /* reset temporal position: the rank in attention order          */
  int32_t reserved;
} lact_key_frame;

/* Bookkeeping counters.  F frames appended; E = max(0, F - W) frames evicted from the
 * window; G groups compressed (group g = frames [r*g, r*g + r)).  Window = frames [E, F);
 * pending = E - r*G evicted frames waiting for a complete group (not attended);
 * memory = groups [max(0, G - M), G) in slots g mod M; raw slot of frame f = f mod R with
 * R = W + B_max + r - 1. */
typedef struct {
  int64_t F, E, G;
  int32_t win_len, mem_len, pending, ring_slots;
  uint64_t version;      /* +1 on every append and on every compress that consumed groups */
  int32_t staged_frames; /* current frames staged by the last lact_rope_reset_apply       */
  int32_t staged_valid;  /* 1 if that staging was done at the present version             */
  int32_t ref_valid;     /* 1 once the reference segment is stored (every member's, in a set) */
  int32_t staged_member; /* member whose operands the staging holds (0 for a single cache)  */
} lact_state;

/* Offsets (bytes, 256-aligned) of the regions inside the cache buffer, so a caller can
 * inspect or snapshot it.  Scale regions, vcur_scale, vscale and vmax are 0-sized unless
 * kv_dtype is
 * FP8_E4M3.  The persistent regions (ring_*, mem_*, ref_* and their scales) come first and
 * are per member: member m's copy of a region starts at offset + m * member_bytes.  The
 * staging regions (krot, qrot, vcur, vcur_scale, vscale, rope_table, attn_flags, vmax)
 * follow all
 * members and are shared by them.
 *   ring_k/ring_v  [R][T][H][D] kv dtype            raw ring (pre-RoPE K, V)
 *   mem_k/mem_v    [M][T][H][D] kv dtype            compressed memory slots
 *   ref_k/ref_v    [ref_frames][T][H][D] kv dtype   reference segment (pre-RoPE K, V)
 *   krot           [H][(ref+M+W+B_max)*T][D] operand  rotated keys in attention order
 *   qrot           [H][B_max*T][D] operand          rotated queries of the block, times
 *                                                   log2(e)/sqrt(D) (the softmax scale
 *                                                   and the change to base 2)
 *   vcur           [B_max][T][H][D] kv dtype        current V staged for attention (FP8:
 *                                                   quantised per (token, head) row as the
 *                                                   cache stores it)
 *   vcur_scale     [B_max][T][H] f32                FP8: the row scales of vcur
 *   vscale         [3][H][(ref+M+W+B_max)*T + 64]   FP8: of every key in attention order
 *                  4 B                              its V row scale s_v (f32), 1/s_v (f32)
 *                                                   and log2(s_v) as a bf16 (hi, lo) pair;
 *                                                   zeros after the last key up to the
 *                                                   next multiple of 64
 *   *_scale        f32 per (token, head): ring/mem/ref [slots][T][H]
 *   rope_table     float2 (cos, sin) table
 *   attn_flags     int32 per (head, 256-row query tile): attention work queue of the exact
 *                  fallback pass (rows whose fast pass could not be trusted)
 *   vmax           [H][32] f32: FP8, partial maxima of each head's V scales
 * The persistent state is ring_*, mem_* and ref_* (and their scales); the rest is rewritten by
 * every step.  operand dtype = q_dtype: an FP8 cache's keys are dequantised (code * scale)
 * and rotated into bf16 by the RoPE pass; its V stays e4m3 and attention multiplies it in
 * on fp8 matrix cores. */
typedef struct {
  size_t total;
  size_t ring_k, ring_v, mem_k, mem_v, ref_k, ref_v, krot, qrot, vcur, vcur_scale, vscale;
  size_t ring_k_scale, ring_v_scale, mem_k_scale, mem_v_scale, ref_k_scale, ref_v_scale;
  size_t rope_table, attn_flags, vmax;
  size_t frame_bytes;    /* T*H*D * kv element size                                       */
  int32_t ring_slots, key_frames_max;
  size_t member_bytes;   /* stride between members' persistent regions                    */
  int32_t members;       /* 1 for a single cache                                          */
  int32_t reserved;
} lact_layout;

typedef struct lact_cache lact_cache; /* opaque host handle */
typedef struct lact_plan lact_plan;   /* opaque host-only bookkeeping planner */

/* ---- sizing -------------------------------------------------------------------------- */

/* Device bytes one cache needs. A pure function of cfg: the footprint never changes with
 * the number of AR steps (walkthrough, "Streaming Pipeline": constant KV size). */
lact_status lact_cache_footprint(const lact_cfg* cfg, size_t* device_bytes);
/* Region offsets of the cache buffer for cfg (see lact_layout). Pure. */
lact_status lact_cache_layout(const lact_cfg* cfg, lact_layout* out);

/* ---- lifetime ------------------------------------------------------------------------ */

/* Binds a caller-owned device buffer of >= lact_cache_footprint bytes (256-byte aligned)
 * to a new host handle. Host work only: nothing is enqueued, nothing is allocated on the
 * device. The buffer contents need no initialisation. */
lact_status lact_cache_init(const lact_cfg* cfg, void* device_buf, size_t bytes, lact_cache** out);
/* Frees the host handle only; the device buffer stays the caller's. NULL is a no-op. */
lact_status lact_cache_destroy(lact_cache* cache);

/* ---- cache sets ------------------------------------------------------------------------ */

/* A set of n_members caches of one cfg, one per (layer, diffusion step): the pages' model
 * keeps a KV cache in every self-attention layer, and under Neighbor Forcing each of the 3
 * distilled denoising steps of a block reuses the KV built at that same step (walkthrough,
 * "Neighbor Forcing", "ConvKV Memory" and "3-step distilled inference"), so all of them
 * append one block and compress once between blocks ("Streaming Pipeline").  The members
 * share one bookkeeping (they always hold the same frames), one staging area and one RoPE
 * table; each has its own ring, memory and reference segment.  Per member, the step is
 * lact_member_rope_reset_apply -> lact_member_block_attention; once per block, for all
 * members, lact_kv_ring_append -> lact_convkv_compress.  1 <= n_members <= LACT_MAX_MEMBERS.
 * A set of 1 is a cache: lact_cache_footprint / layout / init are these with n_members = 1. */
lact_status lact_set_footprint(const lact_cfg* cfg, int32_t n_members, size_t* device_bytes);
lact_status lact_set_layout(const lact_cfg* cfg, int32_t n_members, lact_layout* out);
lact_status lact_set_init(const lact_cfg* cfg, int32_t n_members, void* device_buf, size_t bytes,
                          lact_cache** out);

/* ---- the reference segment ------------------------------------------------------------- */

/* Stores the reference segment: the KV of ref_frames frames (the reference image's part of
 * the context; walkthrough, "ConvKV Memory": reference image, long-term memory, short-term
 * window, current block) that every later step attends first, at the fixed temporal
 * positions 0 .. ref_frames-1 (memory, window and block ranks follow them).  Stored like a
 * ring frame: as given, bf16, or FP8_E4M3 quantised per (token, head).  May be called again
 * to replace it.  Until it has been called, a cache with ref_frames > 0 refuses
 * lact_rope_reset_apply with LACT_E_STATE.
 *   k_ref, v_ref: [n_frames*T][H][D] in q_dtype (pre-RoPE K).  n_frames == ref_frames. */
lact_status lact_ref_set(lact_cache* cache, const void* k_ref, const void* v_ref, int32_t n_frames,
                         void* stream);
/* lact_ref_set for member `member` of a set (0 <= member < n_members).  lact_ref_set,
 * lact_rope_reset_apply and lact_block_attention are these with member 0 and refuse a set
 * of more than one member (LACT_E_INVALID). */
lact_status lact_member_ref_set(lact_cache* cache, int32_t member, const void* k_ref,
                                const void* v_ref, int32_t n_frames, void* stream);

/* ---- the four hot-path calls ----------------------------------------------------------- */

/* RoPE reset + apply (fused).  Positions are reset from the present state (press release,
 * technical-principle paragraph: RoPE Reset; news summary, ConvKV Memory bullet):
 * reference frame i -> t = i; memory rank j -> t = ref + j; window rank k ->
 * t = ref + mem_len + k; current frame i -> t = ref + mem_len + win_len + i (ref =
 * ref_frames); (h, w) = the token's grid cell.  Rotation of interleaved channel pairs
 * (2i, 2i+1) of each part by pos * theta^(-2i/d_part).
 * Writes krot (reference + memory + window + current keys) and qrot in the operand dtype
 * (q_dtype).  A BF16 or F32 cache copies no V: the attention reads the block's V in v_cur
 * itself, which must therefore stay unchanged until the lact_block_attention call that
 * follows has run on the stream (the same V goes to lact_kv_ring_append after it).  The
 * stored history keys are read
 * as stored (FP8_E4M3: code * per-(token, head) scale; the model card's FP8 KV cache option
 * keeps K/V in FP8 and dequantises them for use).  An FP8 cache's V stays in e4m3 for the
 * attention: the pass quantises the block's V per (token, head) row as the cache stores it
 * (vcur, vcur_scale), then writes every key's V row scale terms to vscale in attention
 * order and, per head, partial maxima of those scales to vmax.  The history part is rebuilt only when the state changed
 * since the last call.  A call made while `stream` is being captured into a HIP graph records the
 * history rebuild (and the cache's one-time cos/sin table) every time, so each replay
 * stages everything itself, and leaves both marked absent for the next eager call.
 *   q, k_cur, v_cur: [n_frames*T][H][D] in q_dtype.  1 <= n_frames <= B_max. */
lact_status lact_rope_reset_apply(lact_cache* cache, const void* q, const void* k_cur,
                                  const void* v_cur, int32_t n_frames, void* stream);
/* lact_rope_reset_apply for one member of a set: stages that member's operands in the
 * shared staging area (the history part is rebuilt unless the staging already holds this
 * member's history at the present state). */
lact_status lact_member_rope_reset_apply(lact_cache* cache, int32_t member, const void* q,
                                         const void* k_cur, const void* v_cur, int32_t n_frames,
                                         void* stream);

/* Block attention over the staged operands (walkthrough, "Neighbor Forcing": block-wise
 * causal mask of block size m; "ConvKV Memory": the [reference | memory | window | current]
 * context).  O = softmax(Q K^T / sqrt(D) + mask) V per head; every reference, memory and
 * window key is visible; current key j is visible to query i iff block(j) <= block(i).
 *   q_block_frames: HOST array of n_q_blocks block sizes in frames, summing to the staged
 *                   frame count; NULL means one block of all staged frames.
 *   out: [n*T][H][D] in q_dtype.  lse: [H][n*T] f32 natural-log log-sum-exp, or NULL.
 * The block's V is read from the v_cur of the RoPE call (BF16, F32 caches) or from its
 * staged e4m3 codes (FP8_E4M3).
 * LACT_E_STATE unless lact_rope_reset_apply ran at the present state version. */
lact_status lact_block_attention(lact_cache* cache, const int32_t* q_block_frames,
                                 int32_t n_q_blocks, void* out, float* lse, void* stream);
/* lact_block_attention for one member of a set: LACT_E_STATE unless the last RoPE call
 * staged this member at the present state version. */
lact_status lact_member_block_attention(lact_cache* cache, int32_t member,
                                        const int32_t* q_block_frames, int32_t n_q_blocks,
                                        void* out, float* lse, void* stream);

/* Append-only ring append (walkthrough, "ConvKV Memory" and "Streaming Pipeline": only the
 * new tokens' KV are added, cached KV stay unchanged).  Frame F + i goes to raw slot
 * (F + i) mod R; F += n_frames.  FP8_E4M3 quantises per (token, head): scale = amax/448
 * (1 if amax = 0), code = e4m3(x * (448/amax)) rounded to nearest even, saturating.
 *   k_new, v_new: [n_frames*T][H][D] in q_dtype (pre-RoPE K).  1 <= n_frames <= B_max.
 *   For a set: [n_members][n_frames*T][H][D], member after member; one launch appends the
 *   block to every member.
 * LACT_E_STATE if pending >= r (compress first). */
lact_status lact_kv_ring_append(lact_cache* cache, const void* k_new, const void* v_new,
                                int32_t n_frames, void* stream);

/* ConvKV compression (news summary, ConvKV Memory bullet: 1D convolution at 5:1 into a
 * fixed-length memory; press release: rolling compression at a fixed ratio; arXiv listing,
 * Figure 3 caption).  Every complete group g of r evicted frames is compressed, once, into
 * memory slot g mod M, for K and V with their own weights:
 *   m[u][c] = fma chain: acc = b[c]; for k = 0..r-1: acc = fmaf(w[c][k], x_{r*g+k}[u][c], acc)
 * in f32 (x is the stored value, dequantised for FP8), then stored in kv_dtype (FP8:
 * re-quantised per (token, head)).  Groups that a later group of the same call would
 * overwrite (more than M ready at once) are consumed without being written.
 *   w_k, w_v: [C][r] f32; b_k, b_v: [C] f32 (device).  slots_written: host, nullable.
 *   For a set: [n_members][C][r] and [n_members][C] (each member's own conv weights); one
 *   launch per 16 groups compresses every member.
 * With M = 0 ready groups are consumed and dropped (window-only context). */
lact_status lact_convkv_compress(lact_cache* cache, const float* w_k, const float* b_k,
                                 const float* w_v, const float* b_v, void* stream,
                                 int32_t* slots_written);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation) and so cannot rely on any workspace
 * beyond the buffers they pass: lact_member_block_attention with the exact pass's work
 * queue (one int32 per (head, 256-row query tile)) held by the library in a static device
 * array of LACT_STATIC_QUEUE_MAX entries (64 KiB; each GPU the library runs on holds its
 * own copy until the process ends) instead of the cache buffer's attn_flags region.
 * Same arguments, checks, kernels and results as lact_member_block_attention.  It calls
 * no allocator; its first call on a device looks the array's address up (a host-side
 * runtime query, nothing is enqueued).  LACT_E_CAPACITY if heads * ceil(staged frames *
 * T / 256) > LACT_STATIC_QUEUE_MAX.  Every call on one GPU shares that GPU's array, and
 * each launch writes every entry it reads before reading it: calls that overlap on one GPU
 * (streams not ordered with each other) race on the array and must not be issued. */
#define LACT_STATIC_QUEUE_MAX 16384
lact_status lact_member_block_attention_static(lact_cache* cache, int32_t member,
                                               const int32_t* q_block_frames, int32_t n_q_blocks,
                                               void* out, float* lse, void* stream);

/* ---- inspection ------------------------------------------------------------------------ */

lact_status lact_cache_state(const lact_cache* cache, lact_state* out);
/* Key-frame table attention would use for a block of n_cur current frames at the present
 * state (n_cur = 0: memory + window only).  Writes min(cap, count) entries; *n_out = count. */
lact_status lact_cache_keys(const lact_cache* cache, int32_t n_cur, lact_key_frame* out,
                            int32_t cap, int32_t* n_out);

/* ---- host-only planner (the bookkeeping every cache runs; no device, usable anywhere) -- */

lact_status lact_plan_create(const lact_cfg* cfg, lact_plan** out);
lact_status lact_plan_destroy(lact_plan* plan);
/* Same checks and state change as lact_kv_ring_append. */
lact_status lact_plan_append(lact_plan* plan, int32_t n_frames);
/* Same state change as lact_convkv_compress: consumes every complete group.  Writes up to
 * cap consumed group ids (oldest first) to groups (nullable); *n_groups = count consumed;
 * *n_written (nullable) = how many of them are stored (the last min(count, M)). */
lact_status lact_plan_compress(lact_plan* plan, int64_t* groups, int32_t cap, int32_t* n_groups,
                               int32_t* n_written);
lact_status lact_plan_state(const lact_plan* plan, lact_state* out);
lact_status lact_plan_keys(const lact_plan* plan, int32_t n_cur, lact_key_frame* out, int32_t cap,
                           int32_t* n_out);

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* lact_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LACT_H */
