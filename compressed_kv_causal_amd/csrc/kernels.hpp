// kernels.hpp -- argument blocks and host launchers of the gfx950 kernels (shared by the
// C ABI in lact_abi.cpp and the kernel sources).  No kernel code here.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "lact.h"

namespace lact {

enum : int32_t { DT_F32 = LACT_F32, DT_BF16 = LACT_BF16, DT_FP8 = LACT_FP8_E4M3 };

constexpr int kMaxGroupsPerLaunch = 16;

// Where history key frame fi (attention order [reference | memory | window]) lives:
// reference frame i < ref_len is reference slot i; memory rank j is in memory slot
// (mem_slot0 + j) mod M (group G - mem_len + j); window rank k is in raw slot
// (ring_slot0 + k) mod R (frame E + k).  mem_slot0 = (G - mem_len) mod M, ring_slot0 = E mod R.
struct HistMap {
  int32_t ref_len, mem_len, win_len, M, R, mem_slot0, ring_slot0;
};

// Append: frame F + i goes to raw slot (slot0 + i) mod R, slot0 = F mod R.  A set's
// members follow each other at fixed byte strides, on the input side and in the cache.
struct RingWriteArgs {
  const void* src[2];      // K, V: [members][n*T][H][D] in in_dtype
  void* ring[2];           // member 0's raw ring bases [R][T][H][D]
  float* ring_scale[2];    // FP8: member 0's [R][T][H]
  int64_t src_mstride;     // bytes between members' inputs
  int64_t ring_mstride;    // bytes between members' rings (and scales)
  int32_t members;
  int32_t slot0, n_frames, R, T, H, D;
  int32_t in_dtype, kv_dtype;
};

// Compress: group g reads raw slots (r*g + k) mod R = (in_slot0 + k) mod R and writes
// memory slot out_slot = g mod M.
// Every member of a set in one launch: member m's ring, memory and scales are at
// + m * mstride bytes, its weights at + m * w_mstride and biases at + m * b_mstride floats.
struct CompressArgs {
  const void* ring[2];
  const float* ring_scale[2];
  void* mem[2];
  float* mem_scale[2];
  const float* w[2];       // [members][C][r]
  const float* b[2];       // [members][C]
  int64_t mstride, w_mstride, b_mstride;
  int32_t members;
  int32_t in_slot0[kMaxGroupsPerLaunch];
  int32_t out_slot[kMaxGroupsPerLaunch];
  int32_t n_groups, r, R, T, H, D;
  int32_t kv_dtype;
};

// RoPE reset + apply: rebuild rotated history keys (if hist_rows) and stage the block.
// krot and qrot are in the operand dtype = in_dtype (the q dtype; an FP8 cache's keys are
// dequantised here).  vcur is in the kv dtype: an FP8 cache's block V is quantised per
// (token, head) row as the cache stores it, its row scales going to vcur_scale.
struct RopeArgs {
  const void* q;
  const void* k_cur;
  const void* v_cur;       // [n*T][H][D] in in_dtype
  const void* ring_k;
  const void* mem_k;
  const void* ref_k;
  const void* ring_v;
  const void* mem_v;
  const void* ref_v;
  const float* ring_k_scale;
  const float* mem_k_scale;
  const float* ref_k_scale;
  const float* ring_v_scale;
  const float* mem_v_scale;
  const float* ref_v_scale;
  void* krot;              // [H][KF*T][D] operand dtype
  void* qrot;              // [H][B_max*T][D]
  void* vcur;              // [B_max][T][H][D] kv dtype
  float* vcur_scale;       // FP8 only: [B_max][T][H]
  const float2* table;
  HistMap hist;
  int32_t hist_rows;       // 1: rebuild history keys (and, FP8, the history V scales)
  int32_t n_cur, T, H, D, grid_h, grid_w, key_frames_max, block_frames_max;
  int32_t rope_mode, split_t, split_h, split_w;
  int32_t in_dtype, kv_dtype;
  float q_scale;           // qrot = RoPE(q) * q_scale, q_scale = log2(e) / sqrt(D)
};

struct RopeTableArgs {
  float2* table;
  int32_t rope_mode, split_t, split_h, split_w, D, T, grid_h, grid_w, key_frames_max;
  double theta;
  int64_t entries;
};

// Attention of the staged block over [reference | memory | window | current] (operand dtype).  The
// staged queries carry the softmax scale and the change to base 2: q . k is already the
// exponent of 2 that softmax(q k / sqrt(D)) takes.
struct AttnArgs {
  const void* q;           // qrot
  const void* k;           // krot
  const void* v_ring;      // V rows of window frames (raw ring slots)
  const void* v_mem;       // V rows of memory frames (memory slots)
  const void* v_ref;       // V rows of reference frames (reference slots)
  const void* v_cur;       // V rows of the block's frames
  // FP8 cache: V rows above are e4m3 codes; the value of key j, head h is code *
  // vscale[h * vs_head_stride + j] (plane 0; plane p at + p * vs_plane); vmax[h * 32 ..
  // h * 32 + 31] are partial maxima of the head's scales
  const float* vscale;
  const float* vmax;
  int64_t vs_head_stride, vs_plane;
  int32_t v_fp8;
  void* out;               // [Lq][H][D] q dtype
  float* lse;              // [H][Lq] or null
  int32_t* flags;          // per (head, 256-row query tile): 1 = redo with the exact pass
  int64_t q_head_stride, k_head_stride;  // elements (= rows * D) between heads
  HistMap hist;
  int32_t T, H, D, Lq, Lk, Lhist;
  int32_t n_blocks;
  int32_t block_end[LACT_MAX_Q_BLOCKS];  // cumulative query-token ends of the blocks
};

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s);
hipError_t launch_ring_write(const RingWriteArgs& a, int64_t rows, hipStream_t s);
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);
// FP8 cache: every key's V row scale s_v in attention order [reference | memory | window |
// block], as 3 planes [H][KF*T + kVscalePad]: s_v, 1/s_v, and log2(s_v) as a bf16 (hi, lo)
// pair, each head's row followed by zeros up to the next multiple of 64 keys (so that the
// attention copies whole 8-key groups of a 64-key tile without a bound check); and
// vmax[h * kVmaxParts + p] = the largest s_v of the p-th of kVmaxParts slices of head h's
// keys (0 for an empty slice).
constexpr int kVmaxParts = 32;
constexpr int kVscalePad = 64;
struct VscaleArgs {
  const float* ring_v_scale;  // [R][T][H]
  const float* mem_v_scale;   // [M][T][H]
  const float* ref_v_scale;   // [ref][T][H]
  const float* vcur_scale;    // [B_max][T][H]
  float* vscale;              // [3][H][KF*T + kVscalePad]
  float* vmax;                // [H][kVmaxParts]
  HistMap hist;
  int32_t T, H, Lk, key_frames_max;
};
hipError_t launch_vscale_stage(const VscaleArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, int32_t op_dtype, hipStream_t s);

}  // namespace lact
