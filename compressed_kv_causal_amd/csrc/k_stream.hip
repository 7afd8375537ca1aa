// k_stream.hip -- the bandwidth-bound kernels of the step, for gfx950:
//   k_ring_write   append-only ring append (+ FP8 row quantisation)
//   k_compress     ConvKV depthwise strided temporal conv, r frames -> one memory slot
//   k_rope_table   cos/sin table of the bounded reset positions (double, once per cache)
//   k_rope         RoPE reset + apply: rotated history keys, rotated block Q/K, staged V
//   k_vscale_stage FP8 cache: every key's V scale terms in attention order
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
// (the channel block), so a wave reads and writes 1 KiB contiguous per token and frame (512
// B for FP8); each workgroup takes one (channel block, run of TOK tokens) item, the items
// laid out over the XCDs so that a token run's channel blocks share one L2;
// blockIdx.z = (member, group, tensor).  D/8 lanes form one (token, head) row, which is
// what the FP8 row quantiser reduces over.
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
// each token's loads in turn).  A workgroup is WY waves on consecutive token runs of one
// channel block: (TOK, WY) = (2, 4) keeps 115 VGPRs (four waves per SIMD) and moved a
// 512x512 group 2 % (bf16) and 6 % (FP8) faster than (4, 1), while (8, 1), (2, 1) and
// (4, 4) were slower or the same.
template <int LPR, int R, int TOK, int WY, int KV>
__global__ __launch_bounds__(64 * WY) void k_compress_r(const CompressArgs a) {
  using Raw = typename std::conditional<KV == DT_FP8, uint2, uint4>::type;  // 8 stored elements
  const int32_t C = a.H * a.D;
  // (channel block, token run) of this workgroup, the head groups of a token run on one
  // XCD (they share the FP8 row scales' cache lines)
  const int32_t item = xcd_item(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * gridDim.y);
  const int32_t bx = item % gridDim.x, by = (item / gridDim.x) * WY + threadIdx.y;
  const int32_t c0 = (bx * 64 + threadIdx.x) * 8;          // first channel of this lane
  if (c0 >= C) return;                                     // whole LPR groups leave together
  const CompressPtrs p = compress_ptrs(a);
  const int gi = p.gi;
  const int32_t u0 = by * TOK;
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

// cos/sin of the 4 pairs of one lane (channels 8*li .. 8*li+7) at temporal position t of
// token u, whose grid row and column are gr and gc (3D mode; all three are wave-uniform, so
// the table index is a select and an add per pair, with no division).
__device__ __forceinline__ void rope_cs(const RopeArgs& a, int32_t t, int32_t u, int32_t gr, int32_t gc,
                                        int li, float2* cs) {
  const int32_t ht = a.split_t / 2, hh = a.split_h / 2, hw = a.split_w / 2;
  const int32_t base_t = t * ht;
  const int32_t base_r = a.key_frames_max * ht + gr * hh - ht;
  const int32_t base_c = a.key_frames_max * ht + a.grid_h * hh + gc * hw - ht - hh;
  const int64_t base_1d = ((int64_t)t * a.T + u) * (a.D / 2);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int32_t pair = li * 4 + p;
    if (a.rope_mode == 1)
      cs[p] = a.table[base_1d + pair];
    else
      cs[p] = a.table[(pair < ht ? base_t : (pair < ht + hh ? base_r : base_c)) + pair];
  }
}

__device__ __forceinline__ void rope_rotate8(const float2* cs, float* x) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float x0 = x[2 * p], x1 = x[2 * p + 1];
    x[2 * p] = x0 * cs[p].x - x1 * cs[p].y;
    x[2 * p + 1] = x0 * cs[p].y + x1 * cs[p].x;
  }
}

// blockIdx.y = key frame: frames [0, n_hist) are history frames of [reference | memory | window],
// rotated at t = fi into krot[h][fi*T + u] (only when the history is rebuilt, else the grid
// starts at the block's frames); frames after are the block's frames i = fi - n_hist at
// t = fi: q -> qrot (times q_scale = log2(e)/sqrt(D), so that q . k is the base-2 exponent
// of the softmax), k -> krot[h][t*T + u].  krot and qrot are in the operand dtype
// (in_dtype); an FP8 cache's keys are read as code * row scale.  V is never copied as it
// is: history V is read by the attention where the cache stores it, and so is the block's
// V of a bf16 or f32 cache, in the caller's buffer (the same layout and dtype).  An FP8
// cache's attention reads V as e4m3 codes, so the pass quantises the block's V like the
// cache will store it (codes to vcur, row scales to vcur_scale).
//
// Work split: blockIdx.x = a run of TPB tokens, so the tokens and their grid coordinates
// are scalars; the workgroup's lanes cover a token's H x D/8 chunks (LPR consecutive lanes
// per head, a wave reads 64 x 16 B contiguous).  A lane issues the history loads of all
// TPB tokens, and a block frame's Q, K and V loads of one token, before the stores that
// use them (the compiler must otherwise assume the stores may alias them).
template <int LPR, int TPB, int IN, int KV>
__global__ __launch_bounds__(1024) void k_rope(const RopeArgs a) {
  const int32_t rows = a.T * a.H;
  const int32_t n_hist = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  const int32_t fi = blockIdx.y + (a.hist_rows ? 0 : n_hist);
  const int64_t KFT = (int64_t)a.key_frames_max * a.T;
  const int64_t QT = (int64_t)a.block_frames_max * a.T;
  const int64_t D = a.D;
  constexpr bool fp8 = KV == DT_FP8;
  int32_t u[TPB], gr[TPB], gc[TPB];
  bool ok[TPB];
#pragma unroll
  for (int t = 0; t < TPB; ++t) {
    const int32_t uu = blockIdx.x * TPB + t;
    ok[t] = uu < a.T;
    u[t] = ok[t] ? uu : a.T - 1;                           // a tail token repeats the last's loads
    gr[t] = a.rope_mode == 1 ? 0 : u[t] / a.grid_w;
    gc[t] = a.rope_mode == 1 ? 0 : u[t] - gr[t] * a.grid_w;
  }
  if (fi < n_hist) {
    int32_t slot;
    const int32_t src = hist_src(a.hist, fi, &slot);
    const void* ksrc = src == SRC_REF ? a.ref_k : (src == SRC_MEM ? a.mem_k : a.ring_k);
    const float* kscale = src == SRC_REF ? a.ref_k_scale : (src == SRC_MEM ? a.mem_k_scale : a.ring_k_scale);
    for (int32_t e = threadIdx.x; e < a.H * LPR; e += blockDim.x) {
      const int32_t h = e / LPR, li = e % LPR;
      float x[TPB][8];
      float2 cs[TPB][4];
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        const int64_t srow = (int64_t)slot * rows + (int64_t)u[t] * a.H + h;
        const float sc = fp8 ? kscale[srow] : 1.0f;
        load8_kv(ksrc, KV, srow * D + li * 8, sc, x[t]);
        rope_cs(a, fi, u[t], gr[t], gc[t], li, cs[t]);
      }
#pragma unroll
      for (int t = 0; t < TPB; ++t) {
        if (!ok[t]) continue;
        rope_rotate8(cs[t], x[t]);
        store8_op(a.krot, IN, (h * KFT + (int64_t)fi * a.T + u[t]) * D + li * 8, x[t]);
      }
    }
    return;
  }
  const int32_t i = fi - n_hist;                           // frame inside the block
  for (int32_t e = threadIdx.x; e < a.H * LPR; e += blockDim.x) {
    const int32_t h = e / LPR, li = e % LPR;
#pragma unroll
    for (int t = 0; t < TPB; ++t) {                        // block frames: one token at a time
      if (!ok[t]) continue;                                // uniform over the workgroup
      const int64_t crow = (int64_t)i * rows + (int64_t)u[t] * a.H + h;  // block [n*T][H][D]
      float xq[8], xk[8], xv[8];
      float2 cs[4];
      load8_in(a.q, IN, crow * D + li * 8, xq);
      load8_in(a.k_cur, IN, crow * D + li * 8, xk);
      if (fp8) load8_in(a.v_cur, IN, crow * D + li * 8, xv);
      rope_cs(a, fi, u[t], gr[t], gc[t], li, cs);
      rope_rotate8(cs, xq);
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) xq[e2] *= a.q_scale;
      store8_op(a.qrot, IN, (h * QT + (int64_t)i * a.T + u[t]) * D + li * 8, xq);
      rope_rotate8(cs, xk);
      store8_op(a.krot, IN, (h * KFT + (int64_t)fi * a.T + u[t]) * D + li * 8, xk);
      if (fp8) {
        const float sc = store8_kv<LPR>(a.vcur, DT_FP8, crow * D + li * 8, xv);
        if (li == 0) a.vcur_scale[crow] = sc;
      }
    }
  }
}

// FP8 attention's per-key V scale terms, in attention order (see VscaleArgs): workgroup
// (h, p) takes the p-th of kVmaxParts slices of head h's keys, reads each key's row scale
// where the cache keeps it (reference, memory or ring slot; the staged block) and writes
// s_v, 1/s_v and the bf16 (hi, lo) split of log2(s_v), contiguous per head, and the
// slice's largest s_v; the last slice's workgroup also writes each plane's zero pad from
// Lk up to the next multiple of 64 (1/s_v = 0 and log2 = 0 there: those keys are masked,
// their probabilities 0).  The attention scales its probabilities by 2^-E_h, 2^E_h the power
// of two above the head's largest s_v, so that probability times s_v stays inside e4m3's
// range, and adds the log2 pair to its scores.  An s_v below the smallest normal f32 (a
// row of all but zero values) counts as that normal in the 1/s_v and log2 planes, where
// it only has to give P~ = 0 and a finite 1/s_v.
__global__ __launch_bounds__(256) void k_vscale_stage(const VscaleArgs a) {
  // (head, slice) of this workgroup: all heads of a slice on one XCD, since they gather from
  // the same cache lines of the [slot][T][H] row scales
  const int32_t item = xcd_item(blockIdx.x + a.H * blockIdx.y, a.H * kVmaxParts);
  const int32_t h = item % a.H, part = item / a.H;
  const int32_t per = (a.Lk + kVmaxParts - 1) / kVmaxParts;
  const int32_t j0 = part * per;
  const int32_t j1 = j0 + per < a.Lk ? j0 + per : a.Lk;
  const int32_t nh = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  const int64_t row = (int64_t)a.key_frames_max * a.T + kVscalePad;
  const int64_t P = (int64_t)a.H * row;
  float* s0 = a.vscale + (int64_t)h * row;
  float m = 0.0f;
  for (int32_t j = j0 + threadIdx.x; j < j1; j += 256) {
    const int32_t fi = j / a.T, u = j - fi * a.T;
    float sv;
    if (fi < nh) {
      int32_t slot;
      const int32_t src = hist_src(a.hist, fi, &slot);
      const float* base = src == SRC_REF ? a.ref_v_scale : (src == SRC_MEM ? a.mem_v_scale : a.ring_v_scale);
      sv = base[((int64_t)slot * a.T + u) * a.H + h];
    } else {
      sv = a.vcur_scale[((int64_t)(fi - nh) * a.T + u) * a.H + h];
    }
    m = fmaxf(m, sv);
    const float sn = fmaxf(sv, 0x1p-126f);
    const float l = log2f(sn);
    const uint16_t hi = f32_to_bf16(l);
    const uint16_t lo = f32_to_bf16(l - bf16_to_f32(hi));
    s0[j] = sv;
    s0[P + j] = 1.0f / sn;
    reinterpret_cast<uint32_t*>(s0)[2 * P + j] = (uint32_t)hi | ((uint32_t)lo << 16);
  }
  if (part == kVmaxParts - 1) {  // the zero pad after the last key
    const int32_t lkp = (a.Lk + 63) / 64 * 64;
    for (int32_t j = a.Lk + threadIdx.x; j < lkp; j += 256) {
      s0[j] = 0.0f;
      s0[P + j] = 0.0f;
      reinterpret_cast<uint32_t*>(s0)[2 * P + j] = 0u;
    }
  }
  m = group_max<64>(m);
  __shared__ float wmax[4];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    a.vmax[h * kVmaxParts + part] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
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
  constexpr int TOK = 2, WY = 4;
  // token runs past T (the last workgroup's upper waves) load the last token and store nothing
  const dim3 grid_r((chunks + 63) / 64, (a.T + TOK * WY - 1) / (TOK * WY), 2 * a.n_groups * a.members);
  if (a.D == 128 && a.r == 5 && a.kv_dtype != DT_F32) {
    if (a.kv_dtype == DT_BF16)
      hipLaunchKernelGGL((k_compress_r<16, 5, TOK, WY, DT_BF16>), grid_r, dim3(64, WY), 0, s, a);
    else
      hipLaunchKernelGGL((k_compress_r<16, 5, TOK, WY, DT_FP8>), grid_r, dim3(64, WY), 0, s, a);
    return hipGetLastError();
  }
  if (a.D == 64 && a.r == 5 && a.kv_dtype != DT_F32) {
    if (a.kv_dtype == DT_BF16)
      hipLaunchKernelGGL((k_compress_r<8, 5, TOK, WY, DT_BF16>), grid_r, dim3(64, WY), 0, s, a);
    else
      hipLaunchKernelGGL((k_compress_r<8, 5, TOK, WY, DT_FP8>), grid_r, dim3(64, WY), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((chunks + 63) / 64, (a.T + 15) / 16, 2 * a.n_groups * a.members);
  if (a.D == 128)
    hipLaunchKernelGGL(k_compress<16>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(k_compress<8>, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_vscale_stage(const VscaleArgs& a, hipStream_t s) {
  if (a.H <= 0 || a.Lk <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_vscale_stage, dim3(a.H, kVmaxParts), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  const int32_t n_hist = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  const int32_t frames = (a.hist_rows ? n_hist : 0) + a.n_cur;
  if (frames <= 0) return hipSuccess;
  // one workgroup per token: H x D/8 lanes, rounded up to whole waves (at most 1024; more
  // heads loop)
  const int64_t lanes = (int64_t)a.H * (a.D / 8);
  const int threads = lanes >= 1024 ? 1024 : (int)((lanes + 63) / 64 * 64);
  constexpr int TPB = 2;
  dim3 grid((a.T + TPB - 1) / TPB, frames);
  // dtypes at compile time: a load's conversion inside a runtime dtype branch makes the
  // compiler wait for that load at once, so a block frame's Q, K, V loads would not overlap
#define LACT_ROPE(L, I, K) hipLaunchKernelGGL((k_rope<L, TPB, I, K>), grid, dim3(threads), 0, s, a)
  const bool d128 = a.D == 128;
  if (a.in_dtype == DT_F32 && a.kv_dtype == DT_F32) {
    if (d128) LACT_ROPE(16, DT_F32, DT_F32); else LACT_ROPE(8, DT_F32, DT_F32);
  } else if (a.in_dtype == DT_BF16 && a.kv_dtype == DT_BF16) {
    if (d128) LACT_ROPE(16, DT_BF16, DT_BF16); else LACT_ROPE(8, DT_BF16, DT_BF16);
  } else if (a.in_dtype == DT_BF16 && a.kv_dtype == DT_FP8) {
    if (d128) LACT_ROPE(16, DT_BF16, DT_FP8); else LACT_ROPE(8, DT_BF16, DT_FP8);
  } else {
    return hipErrorNotSupported;
  }
#undef LACT_ROPE
  return hipGetLastError();
}

}  // namespace lact
