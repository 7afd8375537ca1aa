// k_stream.hip -- the bandwidth-bound kernels of the step, for gfx950:
//   k_ring_write   append-only ring append (+ FP8 row quantisation)
//   k_compress     ConvKV depthwise strided temporal conv, r frames -> one memory slot
//   k_rope_table   cos/sin table of the bounded reset positions (double, once per cache)
//   k_rope         RoPE reset + apply: rotated history keys, rotated block Q/K, staged V
//
// Work unit everywhere: one (token, head) row of D channels, handled by D/8 consecutive
// lanes, 8 channels (16 bytes of bf16) per lane, so a wave reads and writes 64 x 16 B
// contiguous segments; FP8 row scales come from a reduction over the row's lanes.
#include <type_traits>

#include "dev_common.hpp"

namespace lact {

// ---------------------------------------------------------------------------------------
// Append (walkthrough "SoulX-LiveAct", sections "ConvKV Memory" and "Streaming Pipeline":
// cached KV stay unchanged, only the new block's KV are added).
// ---------------------------------------------------------------------------------------
template <int LPR>
__global__ __launch_bounds__(256) void k_ring_write(const RingWriteArgs a) {
  // blockIdx.y = frame of the block, blockIdx.z = (member, tensor K or V); rows of a frame
  // are (token, head) pairs, LPR lanes each
  const int32_t e = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  const int32_t rows = a.T * a.H;
  const int32_t row = e / LPR, li = e % LPR;
  if (row >= rows) return;
  const int32_t fi = blockIdx.y, tensor = blockIdx.z & 1, m = blockIdx.z >> 1;
  const void* src = static_cast<const char*>(a.src[tensor]) + m * a.src_mstride;
  void* ring = static_cast<char*>(a.ring[tensor]) + m * a.ring_mstride;
  int32_t slot = a.slot0 + fi;
  if (slot >= a.R) slot -= a.R;
  const int64_t srow = (int64_t)fi * rows + row;
  const int64_t drow = (int64_t)slot * rows + row;
  float x[8];
  load8_in(src, a.in_dtype, srow * a.D + li * 8, x);
  const float s = store8_kv<LPR>(ring, a.kv_dtype, drow * a.D + li * 8, x);
  if (a.kv_dtype == DT_FP8 && li == 0)
    reinterpret_cast<float*>(reinterpret_cast<char*>(a.ring_scale[tensor]) + m * a.ring_mstride)[drow] = s;
}

// ---------------------------------------------------------------------------------------
// ConvKV compression (news summary "SoulX-LiveAct - Soul App ...", technical principle,
// ConvKV Memory bullet: 1D convolution at 5:1 into a fixed-length memory; arXiv listing,
// Figure 3 caption: lightweight 1D convolution of the long-term KV).  Per (token u,
// channel c): acc = b[c]; acc = fmaf(w[c][k], x_k[u][c], acc) for k = 0..r-1, in f32,
// then stored in the cache dtype.  Each input frame is read once.
// ---------------------------------------------------------------------------------------
// Work split: a workgroup is one wave; lane = one 8-channel chunk of 64 consecutive chunks
// (blockIdx.x), so a wave reads and writes 1 KiB contiguous per token and frame (512 B for
// FP8); blockIdx.y = a run of TOK tokens, blockIdx.z = (member, group, tensor).  D/8 lanes
// form one (token, head) row, which is what the FP8 row quantiser reduces over.
struct CompressPtrs {
  const char* ring;
  const float* ring_scale;
  char* mem;
  float* mem_scale;
  const float* w;
  const float* b;
  int gi;
};

// blockIdx.z -> the group and this member's tensors
__device__ __forceinline__ CompressPtrs compress_ptrs(const CompressArgs& a) {
  const int tensor = blockIdx.z & 1;
  const int mg = blockIdx.z >> 1;
  const int m = mg / a.n_groups;
  CompressPtrs p;
  p.gi = mg - m * a.n_groups;
  const int64_t mb = m * a.mstride;
  p.ring = static_cast<const char*>(a.ring[tensor]) + mb;
  p.mem = static_cast<char*>(a.mem[tensor]) + mb;
  p.ring_scale = nullptr;
  p.mem_scale = nullptr;
  if (a.kv_dtype == DT_FP8) {
    p.ring_scale = reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.ring_scale[tensor]) + mb);
    p.mem_scale = reinterpret_cast<float*>(reinterpret_cast<char*>(a.mem_scale[tensor]) + mb);
  }
  p.w = a.w[tensor] + m * a.w_mstride;
  p.b = a.b[tensor] + m * a.b_mstride;
  return p;
}
//
// k_compress_r: the ratio is a compile-time R.  The lane keeps its 8 x R weights and 8
// biases in registers and issues every load of its TOK tokens x R frames before the first
// use, so a wave has TOK * R * 1 KiB in flight (a store to the memory slot cannot alias
// the ring in this kernel, but the compiler cannot know that and would otherwise wait for
// each token's loads in turn).
template <int LPR, int R, int TOK, int KV>
__global__ __launch_bounds__(64) void k_compress_r(const CompressArgs a) {
  using Raw = typename std::conditional<KV == DT_FP8, uint2, uint4>::type;  // 8 stored elements
  const int32_t C = a.H * a.D;
  const int32_t c0 = (blockIdx.x * 64 + threadIdx.x) * 8;  // first channel of this lane
  if (c0 >= C) return;                                     // whole LPR groups leave together
  const CompressPtrs p = compress_ptrs(a);
  const int gi = p.gi;
  const int32_t u0 = blockIdx.y * TOK;
  const int32_t rows = a.T * a.H;
  const char* ring = p.ring;
  constexpr int EB = KV == DT_FP8 ? 1 : 2;                 // stored bytes per element

  Raw raw[TOK][R];
  float sc[TOK][R];
  int32_t slot[R];
#pragma unroll
  for (int k = 0; k < R; ++k) {
    slot[k] = a.in_slot0[gi] + k;
    if (slot[k] >= a.R) slot[k] -= a.R;
  }
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    const int32_t u = u0 + t < a.T ? u0 + t : a.T - 1;     // tail tokens repeat the last one
    const int32_t hrow = u * a.H + c0 / (8 * LPR);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int64_t el = (int64_t)slot[k] * a.T * C + (int64_t)u * C + c0;
      raw[t][k] = *reinterpret_cast<const Raw*>(ring + el * EB);
      sc[t][k] = KV == DT_FP8 ? p.ring_scale[(int64_t)slot[k] * rows + hrow] : 1.0f;
    }
  }
  float w[8][R], b[8];
  const float* wp = p.w + (int64_t)c0 * R;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    b[e] = p.b[c0 + e];
#pragma unroll
    for (int k = 0; k < R; ++k) w[e][k] = wp[e * R + k];
  }
#pragma unroll
  for (int t = 0; t < TOK; ++t) {
    const int32_t u = u0 + t;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = b[e];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float x[8];
      if (KV == DT_FP8) {
        e4m3x4_to_f32(raw[t][k].x, x);
        e4m3x4_to_f32(raw[t][k].y, x + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= sc[t][k];
      } else {
        const uint4 v = reinterpret_cast<const uint4&>(raw[t][k]);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32((uint16_t)(wd[e / 2] >> (16 * (e % 2))));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[e][k], x[e], acc[e]);
    }
    if (u >= a.T) continue;        // uniform per LPR group: a row's lanes share u
    const int64_t dst = (int64_t)a.out_slot[gi] * a.T * C + (int64_t)u * C + c0;
    const float s = store8_kv<LPR>(p.mem, KV, dst, acc);
    if (KV == DT_FP8 && (threadIdx.x % LPR) == 0)
      p.mem_scale[(int64_t)a.out_slot[gi] * rows + u * a.H + c0 / (8 * LPR)] = s;
  }
}

// k_compress: any ratio and the f32 cache; tokens one after another.
template <int LPR>
__global__ __launch_bounds__(64) void k_compress(const CompressArgs a) {
  constexpr int TOK = 16;
  const int32_t C = a.H * a.D;
  const int32_t c0 = (blockIdx.x * 64 + threadIdx.x) * 8;  // first channel of this lane
  if (c0 >= C) return;
  const CompressPtrs p = compress_ptrs(a);
  const int gi = p.gi;
  const int32_t r = a.r;
  float b[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = p.b[c0 + e];
  const int32_t u0 = blockIdx.y * TOK;
  for (int32_t u = u0; u < u0 + TOK && u < a.T; ++u) {
    const int64_t el = (int64_t)u * C + c0;                // element offset inside a frame
    const int32_t hrow = u * a.H + c0 / (8 * LPR);         // (token, head) row inside a frame
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = b[e];
    for (int k = 0; k < r; ++k) {
      int32_t slot = a.in_slot0[gi] + k;
      if (slot >= a.R) slot -= a.R;
      const float sc = a.kv_dtype == DT_FP8 ? p.ring_scale[(int64_t)slot * a.T * a.H + hrow] : 1.0f;
      float x[8];
      load8_kv(p.ring, a.kv_dtype, (int64_t)slot * a.T * C + el, sc, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(p.w[(int64_t)(c0 + e) * r + k], x[e], acc[e]);
    }
    const int64_t dst = (int64_t)a.out_slot[gi] * a.T * C + el;
    const float s = store8_kv<LPR>(p.mem, a.kv_dtype, dst, acc);
    if (a.kv_dtype == DT_FP8 && (threadIdx.x % LPR) == 0)
      p.mem_scale[(int64_t)a.out_slot[gi] * a.T * a.H + hrow] = s;
  }
}

// ---------------------------------------------------------------------------------------
// RoPE (press release digi.china.com, technical-principle paragraph: RoPE Reset keeps
// positions aligned and bounded; news summary, ConvKV Memory bullet).  Interleaved pairs
// (2i, 2i+1) of each part, angle = pos * theta^(-2i/d_part).  Positions are bounded by the
// reset (t < M + W + B_max), so every angle comes from a small table computed once in
// double precision and rounded to f32.
//   3D table: [KF][d_t/2] (t) | [grid_h][d_h/2] (row) | [grid_w][d_w/2] (column)
//   1D table: [KF*T][D/2], position t*T + u
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rope_table(const RopeTableArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.entries) return;
  int64_t pos;
  int32_t pair, dpart;
  if (a.rope_mode == 1) {
    const int32_t half = a.D / 2;
    pos = i / half;
    pair = (int32_t)(i % half);
    dpart = a.D;
  } else {
    const int32_t ht = a.split_t / 2, hh = a.split_h / 2, hw = a.split_w / 2;
    const int64_t nt = (int64_t)a.key_frames_max * ht, nh = (int64_t)a.grid_h * hh;
    if (i < nt) {
      pos = i / ht;
      pair = (int32_t)(i % ht);
      dpart = a.split_t;
    } else if (i < nt + nh) {
      pos = (i - nt) / hh;
      pair = (int32_t)((i - nt) % hh);
      dpart = a.split_h;
    } else {
      pos = (i - nt - nh) / hw;
      pair = (int32_t)((i - nt - nh) % hw);
      dpart = a.split_w;
    }
  }
  const double ang = (double)pos * pow(a.theta, -2.0 * (double)pair / (double)dpart);
  a.table[i] = make_float2((float)cos(ang), (float)sin(ang));
}

// Rotates the 4 pairs of one lane (channels 8*li .. 8*li+7) at temporal position t.
__device__ __forceinline__ void rope_rotate8(const RopeArgs& a, int32_t t, int32_t u, int li,
                                             float* x) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int32_t pair = li * 4 + p;
    float2 cs;
    if (a.rope_mode == 1) {
      cs = a.table[((int64_t)t * a.T + u) * (a.D / 2) + pair];
    } else {
      const int32_t ht = a.split_t / 2, hh = a.split_h / 2, hw = a.split_w / 2;
      if (pair < ht) {
        cs = a.table[t * ht + pair];
      } else if (pair < ht + hh) {
        cs = a.table[a.key_frames_max * ht + (u / a.grid_w) * hh + (pair - ht)];
      } else {
        cs = a.table[a.key_frames_max * ht + a.grid_h * hh + (u % a.grid_w) * hw +
                     (pair - ht - hh)];
      }
    }
    const float x0 = x[2 * p], x1 = x[2 * p + 1];
    x[2 * p] = x0 * cs.x - x1 * cs.y;
    x[2 * p + 1] = x0 * cs.y + x1 * cs.x;
  }
}

// blockIdx.y = key frame: frames [0, n_hist) are history frames of [reference | memory | window],
// rotated at t = fi into krot[h][fi*T + u] (only when the history is rebuilt, else the grid
// starts at the block's frames); frames after are the block's frames i = fi - n_hist at
// t = fi: q -> qrot (times q_scale = log2(e)/sqrt(D), so that q . k is the base-2 exponent
// of the softmax), k -> krot[h][t*T + u], v -> vcur.  Every output is in the operand
// dtype (in_dtype).  An FP8 cache is dequantised on the way (code * row scale), and its
// history V rows are dequantised into vhist in attention order as well.
template <int LPR>
__global__ __launch_bounds__(256) void k_rope(const RopeArgs a) {
  const int32_t e = (int32_t)(blockIdx.x * blockDim.x + threadIdx.x);
  const int32_t rows = a.T * a.H;
  const int32_t row = e / LPR, li = e % LPR;              // row = u * H + h inside the frame
  if (row >= rows) return;
  const int32_t u = row / a.H, h = row - u * a.H;
  const int32_t n_hist = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  const int32_t fi = blockIdx.y + (a.hist_rows ? 0 : n_hist);
  const int64_t KFT = (int64_t)a.key_frames_max * a.T;
  const int64_t QT = (int64_t)a.block_frames_max * a.T;
  const int64_t D = a.D;
  const bool fp8 = a.kv_dtype == DT_FP8;
  float x[8];
  if (fi < n_hist) {
    int32_t slot;
    const int32_t src = hist_src(a.hist, fi, &slot);
    const int64_t srow = (int64_t)slot * rows + row;
    const void* ksrc = src == SRC_REF ? a.ref_k : (src == SRC_MEM ? a.mem_k : a.ring_k);
    const float* kscale = src == SRC_REF ? a.ref_k_scale : (src == SRC_MEM ? a.mem_k_scale : a.ring_k_scale);
    const float sc = fp8 ? kscale[srow] : 1.0f;
    load8_kv(ksrc, a.kv_dtype, srow * D + li * 8, sc, x);
    rope_rotate8(a, fi, u, li, x);
    const int64_t drow = h * KFT + (int64_t)fi * a.T + u;
    store8_op(a.krot, a.in_dtype, drow * D + li * 8, x);
    if (fp8) {
      const void* vsrc = src == SRC_REF ? a.ref_v : (src == SRC_MEM ? a.mem_v : a.ring_v);
      const float* vscale = src == SRC_REF ? a.ref_v_scale : (src == SRC_MEM ? a.mem_v_scale : a.ring_v_scale);
      load8_kv(vsrc, DT_FP8, srow * D + li * 8, vscale[srow], x);
      store8_op(a.vhist, a.in_dtype, ((int64_t)fi * rows + row) * D + li * 8, x);
    }
    return;
  }
  const int32_t i = fi - n_hist;                           // frame inside the block
  const int64_t crow = (int64_t)i * rows + row;            // row of the block's [n*T][H][D]
  load8_in(a.q, a.in_dtype, crow * D + li * 8, x);
  rope_rotate8(a, fi, u, li, x);
#pragma unroll
  for (int e2 = 0; e2 < 8; ++e2) x[e2] *= a.q_scale;
  store8_op(a.qrot, a.in_dtype, (h * QT + (int64_t)i * a.T + u) * D + li * 8, x);

  load8_in(a.k_cur, a.in_dtype, crow * D + li * 8, x);
  rope_rotate8(a, fi, u, li, x);
  store8_op(a.krot, a.in_dtype, (h * KFT + (int64_t)fi * a.T + u) * D + li * 8, x);

  load8_in(a.v_cur, a.in_dtype, crow * D + li * 8, x);
  store8_op(a.vcur, a.in_dtype, crow * D + li * 8, x);
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
static inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

hipError_t launch_rope_table(const RopeTableArgs& a, hipStream_t s) {
  if (a.entries <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3(blocks_for(a.entries)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ring_write(const RingWriteArgs& a, int64_t rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int lpr = a.D / 8;
  dim3 grid(blocks_for((int64_t)a.T * a.H * lpr), a.n_frames, 2 * a.members);
  if (a.D == 128)
    hipLaunchKernelGGL(k_ring_write<16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_ring_write<8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n_groups <= 0) return hipSuccess;
  const int32_t chunks = a.H * a.D / 8;
  constexpr int TOK = 4;
  if (a.D == 128 && a.r == 5 && a.kv_dtype != DT_F32) {
    dim3 grid((chunks + 63) / 64, (a.T + TOK - 1) / TOK, 2 * a.n_groups * a.members);
    if (a.kv_dtype == DT_BF16)
      hipLaunchKernelGGL((k_compress_r<16, 5, TOK, DT_BF16>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((k_compress_r<16, 5, TOK, DT_FP8>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  if (a.D == 64 && a.r == 5 && a.kv_dtype != DT_F32) {
    dim3 grid((chunks + 63) / 64, (a.T + TOK - 1) / TOK, 2 * a.n_groups * a.members);
    if (a.kv_dtype == DT_BF16)
      hipLaunchKernelGGL((k_compress_r<8, 5, TOK, DT_BF16>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((k_compress_r<8, 5, TOK, DT_FP8>), grid, dim3(64), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((chunks + 63) / 64, (a.T + 15) / 16, 2 * a.n_groups * a.members);
  if (a.D == 128)
    hipLaunchKernelGGL(k_compress<16>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(k_compress<8>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  const int32_t n_hist = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  const int32_t frames = (a.hist_rows ? n_hist : 0) + a.n_cur;
  if (frames <= 0) return hipSuccess;
  const int lpr = a.D / 8;
  dim3 grid(blocks_for((int64_t)a.T * a.H * lpr), frames);
  if (a.D == 128)
    hipLaunchKernelGGL(k_rope<16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_rope<8>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lact
