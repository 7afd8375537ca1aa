// k_attn.hip -- block attention over [reference | memory | window | current] on gfx950.
//
// O = softmax(Q K^T / sqrt(D) + mask) V per head (walkthrough "SoulX-LiveAct", section
// "ConvKV Memory": context = long-term memory, short-term window, current block; section
// "Neighbor Forcing": block-wise causal mask of block size m).  Memory and window keys are
// visible to every query; current key j is visible to query i iff block(j) <= block(i), so
// query row i sees exactly the key prefix [0, Lhist + block_end[block(i)]).
//
// Kernels:
//   k_attn_bf16_d128_dual  the D = 128 production kernel for a bf16 V (described at its
//                     definition).
//   k_attn_f8v_d128_dual  the D = 128 production kernel for an FP8 cache's e4m3 V (fp8
//                     MFMAs for PV); the key-tile ring of both is described above them.
//   k_attn_bf16<D, F8V>  exact online-softmax flash attention on v_mfma_f32_32x32x16_bf16,
//                     4 waves x 32 query rows, 64-key tiles staged in LDS (K row-major, V
//                     transposed by the staging threads, an FP8 cache's V codes widened to
//                     bf16 there), running max with rescaling: the kernel for D = 64 and
//                     T < 64, and the exact fallback of the D = 128 kernel for the query
//                     tiles it flags.
//   k_attn_f32<D>     plain f32 FMA kernel (one lane per query row) for the f32 cache.
//
// bf16 kernel orientation: S^T = K Q^T (K is the MFMA A operand, Q the B operand), so a
// lane owns one query row (column l%32 of the 32x32 result) and holds 16 of its 32 scores
// per key block; the row max/sum need one exchange with lane l^32.  P^T is then already
// the B operand of O^T = V^T P^T once the key order inside each 16-key group is permuted
// (the A operand rows of K are read in the order perm32 below), and O^T leaves each lane
// with its row's output channels.
#include "dev_common.hpp"

namespace lact {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int32_t block_of_row(const AttnArgs& a, int32_t row) {
  int32_t b = 0;
  while (b < a.n_blocks - 1 && row >= a.block_end[b]) ++b;
  return b;
}

// Element offset of V row (key j, head h).  Key frame fi = j / T of [reference | memory |
// window | current]: history frames are read where they are stored (reference slot,
// memory slot or raw ring), the block's frames from the staged copy.
__device__ __forceinline__ int64_t v_row_off(const AttnArgs& a, int32_t j, int32_t h,
                                             int32_t* which) {
  const int32_t fi = j / a.T;
  const int32_t u = j - fi * a.T;
  const int32_t nh = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  int32_t slot;
  if (fi < nh) {
    *which = hist_src(a.hist, fi, &slot);
  } else {
    slot = fi - nh;
    *which = SRC_CUR;
  }
  return (((int64_t)slot * a.T + u) * a.H + h) * a.D;
}

template <typename T>
__device__ __forceinline__ const T* v_base(const AttnArgs& a, int32_t which) {
  return static_cast<const T*>(which == SRC_MEM ? a.v_mem
                               : which == SRC_RING ? a.v_ring
                               : which == SRC_REF ? a.v_ref : a.v_cur);
}

// Row m of a 32-key block holds actual key perm32(m): bits 2 and 3 swapped.  With this
// order the 8 probabilities a lane holds for a 16-key chunk are 8 consecutive keys.
__device__ __forceinline__ int32_t perm32(int32_t m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// 8 channels of V row (key j, head h) starting at channel d0, as bf16: from bf16 storage,
// or (F8V) e4m3 codes times the key's row scale, rounded to bf16.
template <bool F8V>
__device__ __forceinline__ uint4 v_chunk_bf16(const AttnArgs& a, int32_t j, int32_t h, int d0) {
  int32_t which;
  const int64_t off = v_row_off(a, j, h, &which) + d0;
  if (!F8V) return *reinterpret_cast<const uint4*>(v_base<uint16_t>(a, which) + off);
  float x[8];
  load8_fp8(v_base<uint8_t>(a, which) + off, a.vscale[h * a.vs_head_stride + j], x);
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
  r.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
  return r;
}

template <int D, bool F8V>
__global__ __launch_bounds__(256) void k_attn_bf16(const AttnArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KSTR = D + 8;   // LDS row stride of K (bf16); +16 B keeps ds_read_b128 conflict-free
  constexpr int VSTR = BN + 8;  // LDS row stride of V^T
  constexpr int DC = D / 8;     // 16-byte chunks per row
  __shared__ __align__(16) uint16_t Ks[BN * KSTR];
  __shared__ __align__(16) uint16_t Vt[D * VSTR];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hi = lane >> 5, lr = lane & 31;
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * BM;
  // as the exact fallback of the D = 128 kernel: only the 256-row tiles it flagged
  if (a.flags && a.flags[h * ((a.Lq + 255) / 256) + q0 / 256] == 0) return;
  const int row = q0 + wave * 32 + lr;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)h * a.q_head_stride;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + (int64_t)h * a.k_head_stride;

  bf16x8_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (row < a.Lq)
      qf[kk] = *reinterpret_cast<const bf16x8_t*>(qb + (int64_t)row * D + kk * 16 + hi * 8);
    else
      qf[kk] = bf16x8_t{};
  }
  const int32_t kvis = a.Lhist + a.block_end[block_of_row(a, row < a.Lq ? row : a.Lq - 1)];
  const int32_t last = (q0 + BM < a.Lq ? q0 + BM : a.Lq) - 1;
  const int32_t kend = a.Lhist + a.block_end[block_of_row(a, last)];
  const int32_t kfree = a.Lhist + a.block_end[block_of_row(a, q0)];

  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int k0 = 0; k0 < kend; k0 += BN) {
    // ---- stage K rows and V^T into LDS ----
    for (int c = tid; c < BN * DC; c += 256) {
      const int r = c / DC, col = c - r * DC, j = k0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < a.Lk) v = *reinterpret_cast<const uint4*>(kbase + (int64_t)j * D + col * 8);
      *reinterpret_cast<uint4*>(&Ks[r * KSTR + col * 8]) = v;
    }
    for (int c = tid; c < (BN / 4) * DC; c += 256) {
      const int dchunk = c % DC, quad = c / DC;
      uint4 vv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = k0 + quad * 4 + t;
        vv[t] = make_uint4(0, 0, 0, 0);
        if (j < a.Lk) vv[t] = v_chunk_bf16<F8V>(a, j, h, dchunk * 8);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = half16(vv[0], e) | (half16(vv[1], e) << 16);
        const uint32_t w1 = half16(vv[2], e) | (half16(vv[3], e) << 16);
        *reinterpret_cast<uint2*>(&Vt[(dchunk * 8 + e) * VSTR + quad * 4]) = make_uint2(w0, w1);
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 32-key blocks ----
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const int mrow = kb * 32 + perm32(lr);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&Ks[mrow * KSTR + kk * 16 + hi * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[kk], s[kb], 0, 0, 0);
      }
    }

    // ---- online softmax (exp2 domain) ----
    const bool need_mask = k0 + BN > kfree;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float v = s[kb][j];
        if (need_mask) {
          const int key = k0 + kb * 32 + perm32(((j >> 2) << 3) + (hi << 2) + (j & 3));
          if (key >= kvis) v = -INFINITY;
        }
        s[kb][j] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = exp2f(s[kb][j] - m_use);
        s[kb][j] = p;
        rs += p;
      }
    }
    rs += __shfl_xor(rs, 32);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

    // ---- O^T += V^T P^T, four 16-key chunks ----
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t pf;
#pragma unroll
      for (int t = 0; t < 8; ++t) pf[t] = (__bf16)s[c >> 1][8 * (c & 1) + t];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t vf =
            *reinterpret_cast<const bf16x8_t*>(&Vt[(db * 32 + lr) * VSTR + c * 16 + hi * 8]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  if (row < a.Lq) {
    const float inv = 1.0f / l_run;
    uint16_t* ob = static_cast<uint16_t*>(a.out) + ((int64_t)row * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = db * 32 + jg * 8 + hi * 4;
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(o[db][jg * 4 + 0] * inv) |
              ((uint32_t)f32_to_bf16(o[db][jg * 4 + 1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(o[db][jg * 4 + 2] * inv) |
              ((uint32_t)f32_to_bf16(o[db][jg * 4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(ob + d0) = w;
      }
    }
    if (hi == 0 && a.lse) a.lse[(int64_t)h * a.Lq + row] = (m_run + log2f(l_run)) * 0.6931471805599453f;
  }
}

// ---------------------------------------------------------------------------------------
// The D = 128 key-tile ring of the two production kernels below (T >= 64):
//   * Key tiles of BN = 64 rows are copied global -> LDS with global_load_lds (16 B per
//     lane, no registers) into a ring of NS = 4 stages: the copies of tile j + 3 are in
//     flight while tile j is computed; a constant "s_waitcnt vmcnt + barrier" per tile
//     orders them with the fragment reads (tiles past the end are copied too, clamped, so
//     the count never changes).  bf16 rows (K, and a bf16 cache's V) are stored with an XOR
//     swizzle of their 16-byte chunks:
//         chunk c of key row r sits at position c ^ swz(r), swz(r) = ((r & 3) << 2) | ((r >> 2) & 3)
//     swz is a bijection over 16 consecutive rows (K fragment reads, ds_read_b128 of 16 rows
//     x one chunk, hit 16 distinct 16-byte slots) and puts the low row bits above the chunk
//     bits (a V^T fragment read, ds_read_b64_tr_b16 of 4 rows x 4 chunks per 32 lanes, hits
//     16 distinct slots), so neither read has bank conflicts.  An FP8 cache's e4m3 V rows
//     (128 B) use chunk c ^ (r mod 8) and the 8-bit transposing read (k_attn_f8v_d128_dual).
//   * V^T fragments come from the transposing LDS reads: within each 16-lane group, lanes
//     4t..4t+3 address key row t (16 consecutive channels) and lane i receives channel i
//     of rows 0..3 -- the consecutive keys of one channel the MFMA A operand needs.
//   * Addressing costs almost no VALU work per tile.  Copies: the tile's first key frame
//     and token and the V bases of that frame and the next (memory slot, raw ring slot or
//     staged block frame) are scalar state; a lane adds its constant row offset to one of
//     the two (a 64-key tile spans at most two frames since T >= 64).  Fragment reads: the
//     per-lane LDS offsets of all K and V^T fragments are loop invariants; the ring slot
//     and the fragment's key block or chunk are the instruction's immediate offset, with
//     the free-tile loop unrolled by NS so the slot is a compile-time constant.
//   * Workgroup -> (head, query tile) mapping keeps each XCD (every 8th workgroup id) on
//     the tiles of one head at a time, so that head's K/V stream once through one L2.
// ---------------------------------------------------------------------------------------
namespace d128 {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// One 1 KiB global -> LDS copy per wave (16 B per lane, lane l lands at LDS address
// m0 + 16 l; m0 is wave-uniform).  Issued through inline asm: the compiler then does not
// treat it as an LDS write it must wait for before every later LDS read (it would insert
// vmcnt(0) right after the copy and the prefetch would never overlap); the ring's own
// "s_waitcnt vmcnt + barrier" orders the copies with the reads.  No VGPR is written.
__device__ __forceinline__ void copy_to_lds(const void* src, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}
// The same from a wave-uniform base (an SGPR pair) plus the lane's 32-bit byte offset:
// the address needs no 64-bit add per lane.
__device__ __forceinline__ void copy_to_lds_s(const void* base, unsigned off, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
// The same with 4 B per lane (lane l lands at m0 + 4 l).
__device__ __forceinline__ void copy_dword_to_lds(const void* src, unsigned m0) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The scalars the copies need, as plain values (the kernel's argument block stays in the
// constant kernarg segment: taking a field by a computed offset would make the compiler
// copy the whole block into scratch memory and every use of it per-lane).
struct Geo {
  const char* v_mem;
  const char* v_ring;
  const char* v_cur;
  const char* v_ref;
  int64_t frame_bytes;  // one V frame, T * H * (bytes of a V row)
  int T, Lk, nf, ref_len, mem_end, nh, M, R, mem_slot0, ring_slot0;
  int s_last;           // FP8: first key of the last 8-key group of the zero-padded scale rows
};

// V base address of key frame f of [reference | memory | window | block] (frames past
// the end repeat the last one, so copies issued past the end read finite data inside the
// buffers).
__device__ __forceinline__ const char* frame_base(const Geo& g, int f) {
  f = f < g.nf ? f : g.nf - 1;
  int ms = g.mem_slot0 + (f - g.ref_len);
  ms = ms >= g.M ? ms - g.M : ms;
  int rs = g.ring_slot0 + (f - g.mem_end);
  rs = rs >= g.R ? rs - g.R : rs;
  const char* fb = g.v_ref + f * g.frame_bytes;
  const char* mb = g.v_mem + ms * g.frame_bytes;
  const char* rb = g.v_ring + rs * g.frame_bytes;
  const char* cb = g.v_cur + (f - g.nh) * g.frame_bytes;
  return f < g.ref_len ? fb : (f < g.mem_end ? mb : (f < g.nh ? rb : cb));
}

// Scalar stream state of the copies: frame and token of the first key of the next tile,
// and the V bases of that frame and the next (recomputed when a tile crosses a frame).
struct Stream {
  int f0, u0;
  const char* baseA;
  const char* baseB;
};

// Scheduling fence between pipeline steps (no instruction crosses it): without it the
// compiler moves each MFMA up next to its fragment read and reuses one fragment register,
// exposing the full LDS latency on every MFMA.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

}  // namespace d128

// ---------------------------------------------------------------------------------------
// k_attn_bf16_d128_dual: the D = 128 kernel for a bf16 V (T >= 64).  One wave per SIMD
// (4 waves, 256 query rows per workgroup) and two 32-row query blocks per wave, A and B,
// software-pipelined across key tiles so that every run of MFMAs carries half a softmax:
//
//     X(i): S(i+1) = Q K(i+1)^T - m for A and B (32 MFMAs; each K fragment read feeds two)
//           beside B's exponentials, row sum and bf16 packing of tile i
//     Y(i): O^T += V(i)^T P(i)^T for A and B (32 MFMAs; each V^T fragment read feeds two)
//           beside A's exponentials, row sum and bf16 packing of tile i + 1
//
// Per MFMA step the wave issues one exponential, one add and every other step one packing;
// each K and V^T fragment read from LDS feeds two MFMAs (one per block), half the reads
// of a layout with two 32-row waves per SIMD.  The key tiles come through the ring above.
//   * Softmax against a fixed reference instead of a running maximum: m = the row's
//     largest score over the first key tile plus a margin.  The staged queries carry
//     log2(e)/sqrt(D), and every QK^T chain starts from the broadcast -m instead of 0, so
//     the chain's output is the base-2 exponent of the probability: one v_exp per score,
//     no per-tile rescale of O.  A tile sum that still threatens the f32 range (scores
//     far above m) is not rescaled in place: the wave finishes, a test of its rows'
//     accumulated sums at the end (which any such tile sum passes on to them) makes the
//     workgroup flag its rows in `flags`, and the exact online-softmax kernel redoes
//     them, as it does rows whose l or O came out not finite (margin and threshold at
//     MDELTA, OVF).
//   * The free tiles run in pipelined passes of four (ring slots as compile-time
//     constants); the pass remainder and the tiles that need a per-element mask run
//     unpipelined after them.
// Register use is the point of the layout: O (2 x 64) and the Q fragments (2 x 32) stay in
// AGPRs, the scores, probabilities and addresses in the 256 arch VGPRs.  The MFMAs are
// inline asm so that each operand keeps its register file; a loop with a branch out of
// its passes, or tile state that stays live after the passes, makes the allocator spill,
// hence the flag instead of an early exit and the state handover in (s0, p0) only.
// ---------------------------------------------------------------------------------------
namespace d128dual {

constexpr int D = 128, BM = 256, BN = 64, NS = 4, WAVES = 4;
constexpr int ROW_BYTES = D * 2;
constexpr int TILE_BYTES = BN * ROW_BYTES;  // 16 KiB
constexpr int V_RING = NS * TILE_BYTES;
constexpr int LDS_BYTES = 2 * NS * TILE_BYTES;
constexpr int VMEM_PER_TILE = 8;            // copy instructions per wave per tile: K 4, V 4
constexpr int KAHEAD = 2;                   // K fragment pairs read ahead of their MFMAs
constexpr int VAHEAD = 2;                   // V^T fragments read ahead (each feeds two MFMAs)
// The reference starts MDELTA above the row's largest score of the first tile, and a sum
// of probabilities of OVF = 2^108 or more (a tile's, hence the row's) flags the rows for
// the exact pass: scores up
// to about 108 + MDELTA - 6 above the first tile's largest stay in the kernel (keys with
// outlier channels reach well past 64), the first tile's largest probability is 2^-MDELTA,
// far from f32 underflow, and l and O (at most l times the largest |V|) stay far below
// f32 overflow for any V of ordinary size; a V large enough to overflow O gives a
// non-finite output, which flags the rows too.
constexpr int MDELTA = 56;
constexpr float OVF = 0x1p108f;

using d128::Geo;
using d128::Stream;
using d128::copy_to_lds;
using d128::copy_to_lds_s;
using d128::frame_base;
using d128::step_fence;
using d128::swz;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct Ctx {
  Geo g;
  const char* kbase;  // this head's rotated keys [Lk][128]
  char* lds;
  unsigned lds_u32;
  int wave, lane, hi, lr;
  int kvis[2];        // keys visible to the lane's row of block A / B
  int64_t hrow;       // bytes between consecutive tokens of one V frame
  int crow[4];        // copies: the four 4-row groups of a tile this lane copies
  int koff[4];
  int voff[4];
  int kread[8];       // fragment reads: LDS byte offsets from the ring base (slot 0)
  int vread[4][2];
};

template <int SLOT>
__device__ __forceinline__ int slot_of(int j) { return SLOT >= 0 ? SLOT : j % NS; }

// Copy tile t's 64 key rows of K and V into ring slot t % NS (this wave: rows 16 wave ..
// 16 wave + 15), then advance the stream.
__device__ __forceinline__ void issue(const Ctx& c, int t, Stream& st) {
  const Geo& a = c.g;
  const unsigned slot = (unsigned)(t % NS);
  const unsigned kdst = c.lds_u32 + slot * TILE_BYTES + (unsigned)c.wave * 16 * ROW_BYTES;
  const unsigned vdst = kdst + V_RING;
  if ((t + 1) * BN <= a.Lk) {
    const char* ktile = c.kbase + (int64_t)t * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_to_lds_s(ktile, (unsigned)c.koff[i], kdst + i * 4 * ROW_BYTES);
  } else {  // rows past the last key repeat it
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int key = t * BN + c.crow[i];
      key = key < a.Lk ? key : a.Lk - 1;
      copy_to_lds(c.kbase + (int64_t)key * ROW_BYTES + (c.koff[i] & (ROW_BYTES - 1)), kdst + i * 4 * ROW_BYTES);
    }
  }
  const char* vA = st.baseA + st.u0 * c.hrow;
  if (st.u0 + BN <= a.T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_to_lds_s(vA, (unsigned)c.voff[i], vdst + i * 4 * ROW_BYTES);
  } else {
    const char* vB = st.baseB + (st.u0 - a.T) * c.hrow;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      copy_to_lds((st.u0 + c.crow[i] >= a.T ? vB : vA) + c.voff[i], vdst + i * 4 * ROW_BYTES);
  }
  st.u0 += BN;  // T >= BN: at most one frame boundary per tile
  if (st.u0 >= a.T) {
    st.u0 -= a.T;
    st.f0 += 1;
    st.baseA = st.baseB;
    st.baseB = frame_base(c.g, st.f0 + 1);
  }
}

// The MFMAs.  QK^T: K and Q fragments from AGPRs, scores (destination and accumulator) in
// arch VGPRs, where the exponentials read them.  PV: O in AGPRs for the whole kernel.  The
// compiler does not see inline asm as MFMAs, so it inserts no wait states between them and
// the VALU instructions around them.  They are used only in the pipelined passes, where the
// first VALU read of a score follows the MFMA that last wrote it by three MFMA steps and
// about 25 more instructions (the v_mfma_f32_32x32x16_bf16, 8 passes, needs about 11) and
// no VALU instruction writes an MFMA operand shortly before its MFMA; drain_o separates the
// passes from the builtin MFMAs and VALU uses of O after them.  The generated code is
// checked for this by the tests (tests/asm_hazards.py).
__device__ __forceinline__ f32x16_t qk_first(const bf16x8_t& k, const bf16x8_t& q, const f32x16_t& init) {
  f32x16_t d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "a"(k), "a"(q), "v"(init));
  return d;
}
__device__ __forceinline__ void qk_next(f32x16_t& d, const bf16x8_t& k, const bf16x8_t& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "a"(k), "a"(q));
}
__device__ __forceinline__ void pv_mfma(f32x16_t& o, const bf16x8_t& v, const u32x4_t& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}
// After the inline-asm passes: 24 wait states that every later use of O must follow (O
// passes through the asm, so nothing reading it can be placed before).
__device__ __forceinline__ void drain_o(f32x16_t (&o)[2][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]),
                 "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
}

// Moves a value into AGPRs once (the asm operands then take it without a copy per use).
template <typename T>
__device__ __forceinline__ T in_agprs(T v) {
  T r;
  asm volatile("" : "=a"(r) : "0"(v));
  return r;
}
// Defines the packed probabilities and the sum at this point, so that the code producing
// them stays in the phase it was written in (instead of sinking to where they are used).
__device__ __forceinline__ void pin(u32x4_t (&p)[4], float& sum) {
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) asm volatile("" : "+v"(p[ch]));
  asm volatile("" : "+v"(sum));
}

__device__ __forceinline__ bf16x8_t kfrag(const char* kb, const Ctx& c, int kk, int kb2) {
  return *reinterpret_cast<const bf16x8_t*>(kb + c.kread[kk] + kb2 * 32 * ROW_BYTES);
}

// V^T fragment (16 keys of chunk ch, channels 32 db .. 32 db + 31)
__device__ __forceinline__ bf16x8_t vfrag(const char* vb, const Ctx& c, int ch, int db) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + c.vread[db][0] + ch * 16 * ROW_BYTES));
  const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + c.vread[db][1] + ch * 16 * ROW_BYTES));
  bf16x8_t vf;
  __builtin_memcpy(&vf, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&vf) + 8, &up, 8);
  return vf;
}

// Softmax step e (0..31) of one block's tile: p_e = exp2(s_e) in place (the scores already
// hold q.k - m_ref), the previous step's p into the row sum (so the add never waits on the
// exponential it follows), and at odd e >= 3 the pair (e - 3, e - 2) packed to bf16: pair k
// holds keys 16 (k / 4) + 8 hi + 2 (k mod 4), +1, word k mod 4 of chunk k / 4 of the PV
// operand.
__device__ __forceinline__ void exp_step(f32x16_t (&s)[2], u32x4_t (&p)[4], float& sum, int e) {
  s[e >> 4][e & 15] = __builtin_amdgcn_exp2f(s[e >> 4][e & 15]);
  if (e > 0) sum += s[(e - 1) >> 4][(e - 1) & 15];
  if (e >= 3 && (e & 1)) {
    const int k = (e - 3) >> 1;
    p[k >> 2][k & 3] = pack_bf16x2(s[k >> 3][(2 * k) & 15], s[k >> 3][(2 * k + 1) & 15]);
  }
}
// After step 31: the last value into the sum, the last pair packed.
__device__ __forceinline__ void exp_finish(const f32x16_t (&s)[2], u32x4_t (&p)[4], float& sum) {
  sum += s[1][15];
  p[3][3] = pack_bf16x2(s[1][14], s[1][15]);
}

// X phase on K slot KS: sn[b] = Q_b K(t)^T - m_b for both blocks (from the broadcast
// -m_ref of the rows, negm; INIT0: from 0), beside (EXPB) block B's exponentials of its
// current tile sb, packed into pb, and added to the row sum sumb.  mid() runs after the second MFMA (the
// copies); VS >= 0: the last steps also read the first VAHEAD V^T fragments of the Y phase
// that follows (V slot VS) into vf.  ASM: the inline-asm MFMAs of the pipelined passes;
// otherwise builtins, whose hazards the compiler handles (prologue and tail).
template <int KS, bool EXPB, int VS = -2, bool INIT0 = false, bool ASM = true, typename Mid>
__device__ __forceinline__ void phase_x(const Ctx& c, int t, const bf16x8_t (&qf)[2][8], const f32x16_t (&negm)[2],
                                        f32x16_t (&sn)[2][2], f32x16_t (&sb)[2], u32x4_t (&pb)[4], float& sumb,
                                        bf16x8_t (&vf)[VAHEAD + 1], Mid mid) {
  static_assert(!(ASM && INIT0), "the asm MFMAs start from negm");
  const char* kb = c.lds + slot_of<KS>(t) * TILE_BYTES;
  bf16x8_t kf[KAHEAD + 1][2];
#pragma unroll
  for (int kk = 0; kk < KAHEAD; ++kk) {
    kf[kk][0] = kfrag(kb, c, kk, 0);
    kf[kk][1] = kfrag(kb, c, kk, 1);
  }
  step_fence();
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int blk = m & 1, kb2 = m >> 1;
      if (m == 0 && kk + KAHEAD < 8) {
        kf[(kk + KAHEAD) % (KAHEAD + 1)][0] = kfrag(kb, c, kk + KAHEAD, 0);
        kf[(kk + KAHEAD) % (KAHEAD + 1)][1] = kfrag(kb, c, kk + KAHEAD, 1);
      }
      const bf16x8_t& kfr = kf[kk % (KAHEAD + 1)][kb2];
      if (!ASM)
        sn[blk][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            kfr, qf[blk][kk], kk > 0 ? sn[blk][kb2] : (INIT0 ? f32x16_t{} : negm[blk]), 0, 0, 0);
      else if (kk > 0)
        qk_next(sn[blk][kb2], kfr, qf[blk][kk]);
      else
        sn[blk][kb2] = qk_first(kfr, qf[blk][kk], negm[blk]);
      if (EXPB) exp_step(sb, pb, sumb, 4 * kk + m);
      if (kk == 0 && m == 1) mid();
      if (VS >= 0 && kk == 7 && m < VAHEAD) vf[m] = vfrag(c.lds + VS * TILE_BYTES, c, m >> 2, m & 3);
      step_fence();
    }
  }
  if (EXPB) {
    exp_finish(sb, pb, sumb);
    pin(pb, sumb);
  }
}

// Y phase on V slot VS: o[b] += V^T P_b^T for both blocks from the current tile's packed
// probabilities pc, beside (EXPA) block A's exponentials of the next tile sa, packed into
// pa, and added to the row sum suma.  PRE: the first VAHEAD fragments are already in vf.  ASM: as for
// phase_x.
template <int VS, bool EXPA, bool PRE = false, bool ASM = true>
__device__ __forceinline__ void phase_y(const Ctx& c, int t, const u32x4_t (&pc)[2][4], f32x16_t (&o)[2][4],
                                        f32x16_t (&sa)[2], u32x4_t (&pa)[4], float& suma,
                                        bf16x8_t (&vf)[VAHEAD + 1]) {
  const char* vb = c.lds + slot_of<VS>(t) * TILE_BYTES;
  if (!PRE) {
#pragma unroll
    for (int i = 0; i < VAHEAD; ++i) vf[i] = vfrag(vb, c, i >> 2, i & 3);
  }
  step_fence();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int ch = i >> 2, db = i & 3;
    if (i + VAHEAD < 16) vf[(i + VAHEAD) % (VAHEAD + 1)] = vfrag(vb, c, (i + VAHEAD) >> 2, (i + VAHEAD) & 3);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (ASM)
        pv_mfma(o[b][db], vf[i % (VAHEAD + 1)], pc[b][ch]);
      else
        o[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (VAHEAD + 1)],
                                                           __builtin_bit_cast(bf16x8_t, pc[b][ch]), o[b][db], 0, 0, 0);
      if (EXPA) exp_step(sa, pa, suma, 2 * i + b);
      step_fence();
    }
  }
  if (EXPA) {
    exp_finish(sa, pa, suma);
    pin(pa, suma);
  }
}

// All 32 exponentials of one block's tile, packed, and their sum, unpipelined.
__device__ __forceinline__ float exp_all(f32x16_t (&s)[2], u32x4_t (&p)[4]) {
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    exp_step(s, p, sum, e);
    if ((e & 7) == 7) step_fence();  // keeps the temporaries few
  }
  exp_finish(s, p, sum);
  return sum;
}

__device__ __forceinline__ void mask_tile(f32x16_t (&s)[2], int key0, int hi, int kvis) {
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 32 * kb2 + perm32(((r >> 2) << 3) + (hi << 2) + (r & 3));
      if (key >= kvis) s[kb2][r] = -INFINITY;
    }
}

// True when the lane's accumulated sums reached OVF (or are not finite).  The sums are of
// non-negative terms, so this holds whenever some tile's sum did: the lane's rows met
// scores far above the reference, and the workgroup flags its rows for the exact pass.
// (Tested once at the end instead of after every tile: the test took 4 VALU instructions
// per tile.)
__device__ __forceinline__ bool overflow(const float (&l_part)[2]) {
  return !(l_part[0] < OVF) || !(l_part[1] < OVF);
}

// End of a tile: every copy but the last tile's (VMEM_PER_TILE per wave) has landed, and
// every wave is done with the ring slot the next tile's copy overwrites.
__device__ __forceinline__ void tile_end() {
  static_assert(VMEM_PER_TILE == 8, "the wait count below leaves one tile's copies in flight");
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  __syncthreads();
}

// One pipelined iteration: X on tile i + 1's K (slot KS), Y on tile i's V (slot VS).
// sc: the scores of tile i (block B's not yet exponentiated), sn: tile i + 1's; pc: tile
// i's packed probabilities (A's on entry, B's from X), pn[0]: A's of tile i + 1.  The
// exponentials go straight into the row sums l_part (no per-tile sum is needed).
template <int KS, int VS>
__device__ __forceinline__ void iteration(const Ctx& c, int i, Stream& st, const bf16x8_t (&qf)[2][8],
                                          f32x16_t (&o)[2][4], f32x16_t (&sc)[2][2], f32x16_t (&sn)[2][2],
                                          u32x4_t (&pc)[2][4], u32x4_t (&pn)[2][4], float (&l_part)[2],
                                          const f32x16_t (&negm)[2]) {
  bf16x8_t vf[VAHEAD + 1];
  phase_x<KS, true, VS>(c, i + 1, qf, negm, sn, sc[1], pc[1], l_part[1], vf, [&]() { issue(c, i + NS - 1, st); });
  // Y's first exponentials read scores from X's last MFMA steps: two more wait states keep
  // them the 24 the hazard check asks of every asm MFMA result (the MFMA needs about 11)
  step_fence();
  asm volatile("s_nop 1");
  phase_y<VS, true, true>(c, i, pc, o, sn[0], pn[0], l_part[0], vf);
  tile_end();
}

// Tile i (V in slot 0) after the pipelined passes: block B's exponentials, then PV (A's
// exponentials of tile i are already in l_part[0]).
__device__ __forceinline__ void finish_tile(const Ctx& c, int i, Stream& st, f32x16_t (&o)[2][4],
                                            f32x16_t (&sc)[2][2], u32x4_t (&pc)[2][4], float (&l_part)[2]) {
  issue(c, i + NS - 1, st);
  l_part[1] += exp_all(sc[1], pc[1]);
  bf16x8_t vf[VAHEAD + 1];
  float unused_sum;
  phase_y<0, false, false, false>(c, i, pc, o, sc[0], pc[0], unused_sum, vf);
  tile_end();
}

// One tile (K and V in slot SLOT), unpipelined, with the per-element mask (a no-op for the
// free tiles); s, p: its state.
template <int SLOT>
__device__ __forceinline__ void single_tile(const Ctx& c, int i, Stream& st, const bf16x8_t (&qf)[2][8],
                                            f32x16_t (&o)[2][4], f32x16_t (&s)[2][2], u32x4_t (&p)[2][4],
                                            float (&sum)[2], float (&l_part)[2], const f32x16_t (&negm)[2]) {
  issue(c, i + NS - 1, st);
  f32x16_t unused_s[2];
  u32x4_t unused_p[4];
  bf16x8_t vf[VAHEAD + 1];
  phase_x<SLOT, false, -2, false, false>(c, i, qf, negm, s, unused_s, unused_p, sum[1], vf, []() {});
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    mask_tile(s[b], i * BN, c.hi, c.kvis[b]);
    sum[b] = exp_all(s[b], p[b]);
  }
  l_part[0] += sum[0];
  l_part[1] += sum[1];
  phase_y<SLOT, false, false, false>(c, i, p, o, unused_s, unused_p, sum[0], vf);
  tile_end();
}

}  // namespace d128dual

__global__ __launch_bounds__(256, 1) void k_attn_bf16_d128_dual(const AttnArgs a) {
  using namespace d128dual;
  __shared__ __align__(1024) char lds[LDS_BYTES];

  const int n_qt = (a.Lq + BM - 1) / BM;
  const int item = xcd_item(blockIdx.x, n_qt * a.H);  // one head's tiles on one XCD
  const int h = item / n_qt, qt = item - h * n_qt;

  Ctx c;
  c.g.v_mem = static_cast<const char*>(a.v_mem);
  c.g.v_ring = static_cast<const char*>(a.v_ring);
  c.g.v_cur = static_cast<const char*>(a.v_cur);
  c.g.v_ref = static_cast<const char*>(a.v_ref);
  c.g.frame_bytes = (int64_t)a.T * a.H * ROW_BYTES;
  c.g.T = a.T;
  c.g.Lk = a.Lk;
  c.g.nf = a.Lk / a.T;
  c.g.ref_len = a.hist.ref_len;
  c.g.mem_end = a.hist.ref_len + a.hist.mem_len;
  c.g.nh = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  c.g.M = a.hist.M;
  c.g.R = a.hist.R;
  c.g.mem_slot0 = a.hist.mem_slot0;
  c.g.ring_slot0 = a.hist.ring_slot0;
  c.g.s_last = 0;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.hi = c.lane >> 5;
  c.lr = c.lane & 31;
  c.lds = lds;
  c.lds_u32 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  c.kbase = static_cast<const char*>(a.k) + (int64_t)h * a.k_head_stride * 2;
  c.hrow = (int64_t)a.H * ROW_BYTES;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = c.wave * 16 + i * 4 + (c.lane >> 4);
    const int chunk = (c.lane & 15) ^ swz(r);
    c.crow[i] = r;
    c.koff[i] = r * ROW_BYTES + chunk * 16;
    c.voff[i] = (r * a.H + h) * ROW_BYTES + chunk * 16;
  }
  {
    const int m = perm32(c.lr);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) c.kread[kk] = m * ROW_BYTES + (((2 * kk + c.hi) ^ swz(m)) * 16);
    const int g = c.lane >> 4, i = c.lane & 15;
    const int row = c.hi * 8 + (i >> 2);
    const int half = (i & 1) * 8;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chunk = 4 * db + 2 * (g & 1) + ((i & 3) >> 1);
      c.vread[db][0] = V_RING + row * ROW_BYTES + ((chunk ^ swz(row)) * 16) + half;
      c.vread[db][1] = V_RING + (row + 4) * ROW_BYTES + ((chunk ^ swz(row + 4)) * 16) + half;
    }
  }
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)h * a.q_head_stride;
  const int q0 = qt * BM;
  int rows[2];
  bf16x8_t qf[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    rows[b] = q0 + c.wave * 64 + b * 32 + c.lr;
    const int rr = rows[b] < a.Lq ? rows[b] : a.Lq - 1;
    c.kvis[b] = a.Lhist + a.block_end[block_of_row(a, rr)];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[b][kk] = in_agprs(rows[b] < a.Lq ? *reinterpret_cast<const bf16x8_t*>(qb + (int64_t)rows[b] * D + kk * 16 + c.hi * 8)
                                          : bf16x8_t{});
  }
  const int last = (q0 + BM < a.Lq ? q0 + BM : a.Lq) - 1;
  const int kend = a.Lhist + a.block_end[block_of_row(a, last)];
  const int kfree = a.Lhist + a.block_end[block_of_row(a, q0)];
  const int nt = (kend + BN - 1) / BN;
  const int n_free = kfree / BN;  // >= 1: every row sees at least the first block's T >= 64 keys

  f32x16_t o[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[b][db] = in_agprs(f32x16_t{});
  float m_ref[2], l_part[2] = {0.0f, 0.0f}, sum[2];
  f32x16_t negm[2];
  f32x16_t s0[2][2], s1[2][2];
  u32x4_t p0[2][4], p1[2][4];
  Stream st{0, 0, frame_base(c.g, 0), frame_base(c.g, 1)};
  for (int t = 0; t < NS - 1; ++t) issue(c, t, st);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // tiles 0 and 1 landed
  __syncthreads();

  // tile 0: scores from 0; the reference m_ref = the row's largest; A's exponentials
  {
    bf16x8_t vf[VAHEAD + 1];
    phase_x<0, false, -2, true, false>(c, 0, qf, negm, s0, s1[0], p1[0], sum[1], vf, []() {});
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float mx = fmaxf(s0[b][0][0], s0[b][1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[b][0][r], s0[b][1][r]));
    m_ref[b] = fmaxf(mx, __shfl_xor(mx, 32)) + (float)MDELTA;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      negm[b][r] = -m_ref[b];
      s0[b][0][r] -= m_ref[b];
      s0[b][1][r] -= m_ref[b];
    }
  }
  l_part[0] = exp_all(s0[0], p0[0]);

  // Free tiles, pipelined, in passes of four (the ring slots are compile-time constants;
  // the state alternates between (s0, p0) and (s1, p1) and is back in (s0, p0) after a
  // pass).  A tile sum that overflows is caught by the test of the accumulated sums at the end.
  int i = 0;
  static_assert(NS == 4, "the unrolled loop below walks the slots 0, 1, 2, 3");
  while (i + 4 < n_free) {
    iteration<1, 0>(c, i, st, qf, o, s0, s1, p0, p1, l_part, negm);
    iteration<2, 1>(c, i + 1, st, qf, o, s1, s0, p1, p0, l_part, negm);
    iteration<3, 2>(c, i + 2, st, qf, o, s0, s1, p0, p1, l_part, negm);
    iteration<0, 3>(c, i + 3, st, qf, o, s1, s0, p1, p0, l_part, negm);
    i += 4;
  }
  drain_o(o);
  // tile i (slot 0); then the rest -- the last free tiles and those past n_free, which
  // need the per-element mask -- unpipelined
  finish_tile(c, i, st, o, s0, p0, l_part);
  for (++i; i < nt; ++i) {
    switch (i & 3) {
      case 0: single_tile<0>(c, i, st, qf, o, s0, p0, sum, l_part, negm); break;
      case 1: single_tile<1>(c, i, st, qf, o, s0, p0, sum, l_part, negm); break;
      case 2: single_tile<2>(c, i, st, qf, o, s0, p0, sum, l_part, negm); break;
      default: single_tile<3>(c, i, st, qf, o, s0, p0, sum, l_part, negm); break;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the copies issued past the end

  const bool raised = overflow(l_part);
  int bad = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float l = l_part[b] + __shfl_xor(l_part[b], 32);
    const float inv = 1.0f / l;
    bool ok = l > 0.0f && l < 3.0e38f;
    float outv[4][16];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        outv[db][r] = o[b][db][r] * inv;
        ok = ok && (fabsf(outv[db][r]) < 3.0e38f);
      }
    const int row = rows[b];
    if (row < a.Lq) {
      bad |= (ok && !raised) ? 0 : 1;
      uint16_t* ob = static_cast<uint16_t*>(a.out) + ((int64_t)row * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = db * 32 + jg * 8 + c.hi * 4;
          uint2 w2;
          w2.x = pack_bf16x2(outv[db][jg * 4 + 0], outv[db][jg * 4 + 1]);
          w2.y = pack_bf16x2(outv[db][jg * 4 + 2], outv[db][jg * 4 + 3]);
          *reinterpret_cast<uint2*>(ob + d0) = w2;
        }
      if (c.hi == 0 && a.lse) a.lse[(int64_t)h * a.Lq + row] = (m_ref[b] + log2f(l)) * 0.6931471805599453f;
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0 && a.flags) a.flags[item] = bad;
}


// ---------------------------------------------------------------------------------------
// k_attn_f8v_d128_dual: the D = 128 kernel for an FP8 cache's e4m3 V (T >= 64), in the
// two-block layout of k_attn_bf16_d128_dual (one wave per SIMD, 32-row blocks A and B):
//
//     X(i): S~(i+1) = Q K(i+1)^T + log2 s_v - m for A and B (36 bf16 MFMAs: each chain
//           starts with one 16-channel step that adds the keys' log2 s_v to -m), beside
//           A's e4m3 conversion and B's exponentials, row sum and conversion of tile i
//     Y(i): O^T += V(i)^T P~(i)^T for A and B on the stored e4m3 codes (8 MFMAs of 64
//           keys on v_mfma_scale_f32_32x32x64_f8f6f4) beside A's exponentials and row
//           sum of tile i + 1
//
// P~ = 2^(s + log2 s_v - m) = P' s_v, with P' = 2^(s - m) the probability and s_v the
// key's V row scale, so that the V codes times P~ give P' V.  Instead of a reference that
// is raised when P~ outgrows e4m3, every row scales each tile by its own power of two:
// 2^(E_h + e) bounds the tile's largest P~ (s_v < 2^E_h for every key of the head, and
// the row's sum of P' over the tile's 64 keys, below 2^e, bounds each P'), the codes are
// e4m3(P~ 2^-E) with E = E_h + e - 8, all below 2^8, and the MFMA's E8M0 block scale of
// the P~ operand multiplies 2^E back in.  O is never rescaled: the reference m lies a
// fixed margin above the row's largest s + log2 s_v over the first tile, and only a tile
// sum of P' that threatens f32 range flags the rows for the exact pass (the margin and
// the threshold at the constants MDELTA, OVF).  Key tiles come through the ring above;
// the pipelining, registers and inline-asm MFMAs are those of k_attn_bf16_d128_dual.
// Per ring slot the LDS holds K (16 KiB), the V codes (8 KiB) and the keys' 1/s_v and
// log2 s_v pairs in groups of 8 keys: [8 x 1/s_v | 8 x (hi, lo) bf16] = 64 B per group.
// ---------------------------------------------------------------------------------------
namespace d128dual8 {

constexpr int D = 128, BM = 256, BN = 64, NS = 4, WAVES = 4;
constexpr int ROW_BYTES = D * 2;                 // a bf16 key row
constexpr int TILE_BYTES = BN * ROW_BYTES;       // 16 KiB of keys per ring slot
constexpr int V8_ROW = D;                        // an e4m3 V row
constexpr int V8_TILE = BN * V8_ROW;             // 8 KiB of V codes per slot
constexpr int S_TILE = BN * 8;                   // per slot: 1/s_v and log2 s_v of 64 keys
constexpr int V_RING = NS * TILE_BYTES;
constexpr int S_RING = V_RING + NS * V8_TILE;
constexpr int LDS_BYTES = S_RING + NS * S_TILE;  // 98 KiB
constexpr int VMEM_PER_TILE = 7;                 // copies per wave and tile: K 4, V 2, scales 1
constexpr int KAHEAD = 2;                        // K fragment pairs read ahead of their MFMAs

using d128::Geo;
using d128::Stream;
using d128::copy_dword_to_lds;
using d128::copy_to_lds;
using d128::copy_to_lds_s;
using d128::frame_base;
using d128::lds_v2i32;
using d128::step_fence;
using d128::swz;
using d128::v2i32;
using d128::v8i32;
using d128dual::drain_o;
using d128dual::in_agprs;
using d128dual::MDELTA;
using d128dual::mask_tile;
using d128dual::overflow;
using d128dual::qk_next;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short v2i16 __attribute__((ext_vector_type(2)));

struct Ctx {
  Geo g;
  const char* kbase;   // this head's rotated keys [Lk][128]
  char* lds;
  unsigned lds_u32;
  int wave, lane, hi, lr;
  int kvis[2];         // keys visible to the lane's row of block A / B
  int64_t hrow;        // bytes between consecutive tokens of one V frame (H * 128)
  int crow[4];         // K copies: the four 4-row groups of a tile this lane copies
  int koff[4];
  int vrow[2];         // V copies: the two 8-row groups
  int voff[2];
  int kread[8];        // K fragment reads (LDS byte offsets from the ring base, slot 0)
  int vread[4];        // first of the four 8-key transposed reads of V^T fragment db
  int sread;           // 1/s_v of the lane's keys, chunk 0 (+ 128 B per 8-key chunk)
  int lread[2];        // log2 s_v pair of the A-operand key row of key block kb
  const char* vsbase;  // scale-term copy source of this lane (1/s_v or log2 pairs)
  int eb0;             // E_h - 7
  bf16x8_t augb;       // B operand of the log2 s_v step: bf16 (1, 1) in channels 0, 1
};

template <int SLOT>
__device__ __forceinline__ int slot_of(int j) { return SLOT >= 0 ? SLOT : j % NS; }

// Copy tile t's 64 key rows of K, V codes and V scale terms into ring slot t % NS (this
// wave: rows 16 wave .. 16 wave + 15), then advance the stream.
__device__ __forceinline__ void issue(const Ctx& c, int t, Stream& st) {
  const Geo& a = c.g;
  const unsigned slot = (unsigned)(t % NS);
  const unsigned kdst = c.lds_u32 + slot * TILE_BYTES + (unsigned)c.wave * 16 * ROW_BYTES;
  const unsigned vdst = c.lds_u32 + V_RING + slot * V8_TILE + (unsigned)c.wave * 16 * V8_ROW;
  if ((t + 1) * BN <= a.Lk) {
    const char* ktile = c.kbase + (int64_t)t * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_to_lds_s(ktile, (unsigned)c.koff[i], kdst + i * 4 * ROW_BYTES);
  } else {  // rows past the last key repeat it
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int key = t * BN + c.crow[i];
      key = key < a.Lk ? key : a.Lk - 1;
      copy_to_lds(c.kbase + (int64_t)key * ROW_BYTES + (c.koff[i] & (ROW_BYTES - 1)), kdst + i * 4 * ROW_BYTES);
    }
  }
  const char* vA = st.baseA + st.u0 * c.hrow;
  if (st.u0 + BN <= a.T) {
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_to_lds_s(vA, (unsigned)c.voff[i], vdst + i * 8 * V8_ROW);
  } else {
    const char* vB = st.baseB + (st.u0 - a.T) * c.hrow;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      copy_to_lds((st.u0 + c.vrow[i] >= a.T ? vB : vA) + c.voff[i], vdst + i * 8 * V8_ROW);
  }
  // scale terms of keys 16 wave .. 16 wave + 15: lanes 16 g .. 16 g + 7 the 1/s_v and lanes
  // 16 g + 8 .. 16 g + 15 the log2 pairs of keys 16 wave + 8 g + (lane mod 8).  The planes
  // are zero-padded to a multiple of 64 keys; tiles copied past the end re-read the last group.
  if (c.lane < 32) {
    const int key0 = min(t * BN + c.wave * 16 + (c.lane >> 4) * 8, a.s_last);
    copy_dword_to_lds(c.vsbase + (int64_t)key0 * 4, c.lds_u32 + S_RING + slot * S_TILE + (unsigned)c.wave * 128);
  }
  st.u0 += BN;  // T >= BN: at most one frame boundary per tile
  if (st.u0 >= a.T) {
    st.u0 -= a.T;
    st.f0 += 1;
    st.baseA = st.baseB;
    st.baseB = frame_base(c.g, st.f0 + 1);
  }
}

// The MFMAs beyond k_attn_bf16_d128_dual's (same conventions: scores in VGPRs, O in AGPRs,
// the generated code checked for wait states by the tests).  aug_first starts a QK^T
// chain: d = A B + init with A the key rows' (hi, lo) bf16 pairs of log2 s_v and B = augb.
__device__ __forceinline__ f32x16_t aug_first(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& init) {
  f32x16_t d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(init));
  return d;
}
// O^T += V^T P~^T: 32 channels x 64 keys of e4m3 codes; the P~ operand's block scale is the
// E8M0 byte eb (both 32-key blocks of a column), the V operand's 1.0 (one = 127).
__device__ __forceinline__ void pv_mfma8(f32x16_t& o, const v8i32& v, const v8i32& p, int one, int eb) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(o)
               : "v"(v), "v"(p), "v"(one), "v"(eb));
}

// x + the value of the lane 32 apart (lanes j and j + 32 hold the same query row); the
// wait states are those a VALU write needs before the swap reads its operands.
__device__ __forceinline__ float pair_sum(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

// E8M0 byte 127 + E of a block's tile from the lane's sum of P' (see above), clamped to
// the finite scales (the clamp only ever lowers the codes).  The exponent is read from the
// bits of the row's sum: for a normal sum, frexp's exponent e is its biased exponent field
// minus 126, so 127 + E = 127 + E_h + e - 8 = field + eb0 with eb0 = E_h - 7 (one shift,
// one add and one clamp).  A zero sum (a tile the mask hides from the row: its codes are
// all zero) clamps to 1.
__device__ __forceinline__ int tile_scale(float sum, int eb0) {
  const int e = (int)(__builtin_bit_cast(unsigned, pair_sum(sum)) >> 23) + eb0;
  return min(max(e, 1), 254);
}

// Word w of a block's P~ operand: bytes 4 w .. 4 w + 3 are e4m3(P~ 2^-E) of the values
// 4 w .. 4 w + 3 of s (the byte order of the V^T fragments); eb = 127 + E.
__device__ __forceinline__ void conv_word(const f32x16_t (&s)[2], v8i32& p, int w, int eb) {
  const float scale = __builtin_bit_cast(float, eb << 23);
  const f32x16_t& v = s[w >> 2];
  const int b0 = 4 * (w & 3);
  int x;
  asm volatile("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %5\n\t"
               "v_cvt_scalef32_pk_fp8_f32 %0, %3, %4, %5 op_sel:[0,0,0,1]"
               : "=&v"(x)
               : "v"(v[b0]), "v"(v[b0 + 1]), "v"(v[b0 + 2]), "v"(v[b0 + 3]), "v"(scale));
  p[w] = x;
}

__device__ __forceinline__ bf16x8_t kfrag(const char* kb, const Ctx& c, int kk, int kb2) {
  return *reinterpret_cast<const bf16x8_t*>(kb + c.kread[kk] + kb2 * 32 * ROW_BYTES);
}
// A operand of the log2 s_v step of key block kb: (hi, lo, 0, ...) of the row's key.
__device__ __forceinline__ bf16x8_t aug_frag(const char* sb, const Ctx& c, int kb) {
  const u32x4_t w = {*reinterpret_cast<const uint32_t*>(sb + c.lread[kb]), 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, w);
}
// V^T fragment of channels 32 db .. 32 db + 31 (the lane's 32 keys): four transposing
// 8-bit reads of 8 keys each.
__device__ __forceinline__ v8i32 vfrag(const char* vb, const Ctx& c, int db) {
  v8i32 f;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    const v2i32 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(vb + c.vread[db] + cc * 16 * V8_ROW));
    f[2 * cc] = x[0];
    f[2 * cc + 1] = x[1];
  }
  return f;
}
// 1/s_v of the keys of values 8 ch .. 8 ch + 7 of a block's tile.
__device__ __forceinline__ void read_inv(const char* sb, const Ctx& c, int ch, float (&inv)[8]) {
  const float4 i0 = *reinterpret_cast<const float4*>(sb + c.sread + ch * 128);
  const float4 i1 = *reinterpret_cast<const float4*>(sb + c.sread + ch * 128 + 16);
  inv[0] = i0.x; inv[1] = i0.y; inv[2] = i0.z; inv[3] = i0.w;
  inv[4] = i1.x; inv[5] = i1.y; inv[6] = i1.z; inv[7] = i1.w;
}

// Softmax step e (0..31) of one block's tile: P~_e = exp2(s_e) in place and the previous
// value's P' = P~ / s_v into the row sum (the FMA never waits on the exponential it
// follows); at e = 8 ch the 1/s_v of chunk ch + 1 are read into the buffer chunk ch - 1
// used.  exp_finish adds the last value.
__device__ __forceinline__ void exp_step(const char* sb, const Ctx& c, f32x16_t (&s)[2], float& sum,
                                         float (&inv)[2][8], int e) {
  s[e >> 4][e & 15] = __builtin_amdgcn_exp2f(s[e >> 4][e & 15]);
  if (e > 0) {
    const int f = e - 1;
    sum = __builtin_fmaf(s[f >> 4][f & 15], inv[(f >> 3) & 1][f & 7], sum);
  }
  if ((e & 7) == 0 && e < 24) read_inv(sb, c, (e >> 3) + 1, inv[((e >> 3) + 1) & 1]);
}
__device__ __forceinline__ void exp_finish(const f32x16_t (&s)[2], float& sum, const float (&inv)[2][8]) {
  sum = __builtin_fmaf(s[1][15], inv[1][7], sum);
}

__device__ __forceinline__ void pin(v8i32& p, float& sum) {
  asm volatile("" : "+v"(p));
  asm volatile("" : "+v"(sum));
}

// The softmax work beside X-phase step j (0..35): A's codes (one word per step 0-7), B's
// exponentials (steps 0-31), B's scale (32) and codes (33-35).
__device__ __forceinline__ void soft_x(const Ctx& c, const char* sv, f32x16_t (&sc)[2][2], v8i32 (&pc)[2],
                                       int (&eb)[2], float (&sum)[2], float (&inv)[2][8], int j) {
  if (j < 8) conv_word(sc[0], pc[0], j, eb[0]);
  if (j < 32) exp_step(sv, c, sc[1], sum[1], inv, j);
  if (j == 32) {
    exp_finish(sc[1], sum[1], inv);
    eb[1] = tile_scale(sum[1], c.eb0);
  }
  if (j == 33) {
    conv_word(sc[1], pc[1], 0, eb[1]);
    conv_word(sc[1], pc[1], 1, eb[1]);
    conv_word(sc[1], pc[1], 2, eb[1]);
  }
  if (j == 34) {
    conv_word(sc[1], pc[1], 3, eb[1]);
    conv_word(sc[1], pc[1], 4, eb[1]);
    conv_word(sc[1], pc[1], 5, eb[1]);
  }
  if (j == 35) {
    conv_word(sc[1], pc[1], 6, eb[1]);
    conv_word(sc[1], pc[1], 7, eb[1]);
  }
}

// X phase on slot KS (tile t): sn[b] = Q_b K(t)^T + log2 s_v - m_b for both blocks (from
// the broadcast -m of the rows, negm; INIT0: from 0).  SOFT, beside it (tile t - 1, slot
// VS): block A's codes from its exponentials sc[0] and their sum; block B's exponentials
// of sc[1], their sum, scale and codes.  mid() runs after the sixth MFMA (the copies);
// VS >= 0: the last steps also read the first two V^T fragments of the Y phase into vf.
// ASM: the inline-asm MFMAs of the pipelined passes; otherwise builtins (prologue, tail).
template <int KS, bool SOFT, int VS = -2, bool INIT0 = false, bool ASM = true, typename Mid>
__device__ __forceinline__ void phase_x(const Ctx& c, int t, const bf16x8_t (&qf)[2][8], const f32x16_t (&negm)[2],
                                        f32x16_t (&sn)[2][2], f32x16_t (&sc)[2][2], v8i32 (&pc)[2], int (&eb)[2],
                                        float (&sum)[2], v8i32 (&vf)[2], Mid mid) {
  static_assert(!(ASM && INIT0), "the asm MFMAs start from negm");
  static_assert(!SOFT || VS >= 0, "the softmax reads the scale terms of slot VS");
  const char* kb = c.lds + slot_of<KS>(t) * TILE_BYTES;
  const char* sk = c.lds + slot_of<KS>(t) * S_TILE;
  const char* sv = c.lds + (VS >= 0 ? VS : 0) * S_TILE;
  bf16x8_t kf[KAHEAD + 1][2];
  bf16x8_t ag[2];
  float inv[2][8];
  ag[0] = aug_frag(sk, c, 0);
  ag[1] = aug_frag(sk, c, 1);
  asm volatile("" : "+v"(ag[0]), "+v"(ag[1]));  // built here, not next to their MFMAs
#pragma unroll
  for (int kk = 0; kk < KAHEAD; ++kk) {
    kf[kk][0] = kfrag(kb, c, kk, 0);
    kf[kk][1] = kfrag(kb, c, kk, 1);
  }
  if (SOFT) {
    read_inv(sv, c, 0, inv[0]);
    eb[0] = tile_scale(sum[0], c.eb0);
    sum[1] = 0.0f;
  }
  step_fence();
#pragma unroll
  for (int m = 0; m < 4; ++m) {  // steps 0-3: the log2 s_v steps start the four chains
    const int blk = m & 1, kb2 = m >> 1;
    if (ASM)
      sn[blk][kb2] = aug_first(ag[kb2], c.augb, negm[blk]);
    else
      sn[blk][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ag[kb2], c.augb, INIT0 ? f32x16_t{} : negm[blk], 0, 0, 0);
    if (SOFT) soft_x(c, sv, sc, pc, eb, sum, inv, m);
    step_fence();
  }
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {  // steps 4-35
      const int blk = m & 1, kb2 = m >> 1, j = 4 + 4 * kk + m;
      if (m == 0 && kk + KAHEAD < 8) {
        kf[(kk + KAHEAD) % (KAHEAD + 1)][0] = kfrag(kb, c, kk + KAHEAD, 0);
        kf[(kk + KAHEAD) % (KAHEAD + 1)][1] = kfrag(kb, c, kk + KAHEAD, 1);
      }
      const bf16x8_t& kfr = kf[kk % (KAHEAD + 1)][kb2];
      if (ASM)
        qk_next(sn[blk][kb2], kfr, qf[blk][kk]);
      else
        sn[blk][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr, qf[blk][kk], sn[blk][kb2], 0, 0, 0);
      if (SOFT) soft_x(c, sv, sc, pc, eb, sum, inv, j);
      if (j == 5) mid();
      if (VS >= 0 && (j == 32 || j == 33)) vf[j - 32] = vfrag(c.lds + VS * V8_TILE, c, j - 32);
      step_fence();
    }
  }
  if (SOFT) {
    pin(pc[0], sum[0]);
    pin(pc[1], sum[1]);
  }
}

// Y phase on slot VS (tile t): o[b] += V^T P~_b^T for both blocks, fragment by fragment
// (A, B for channel block db), beside (SOFT) block A's exponentials and row sum of tile
// t + 1 (scores sa, scale terms in slot SA).  PRE: the first two fragments are already in
// vf.  ASM: as for phase_x.
template <int VS, bool SOFT, bool PRE = false, bool ASM = true>
__device__ __forceinline__ void phase_y(const Ctx& c, int t, const v8i32 (&pc)[2], const int (&eb)[2],
                                        f32x16_t (&o)[2][4], f32x16_t (&sa)[2], float& suma, v8i32 (&vf)[2],
                                        int one) {
  constexpr int SA = VS >= 0 ? (VS + 1) % NS : 0;
  const char* vb = c.lds + slot_of<VS>(t) * V8_TILE;
  const char* sb = c.lds + SA * S_TILE;
  float inv[2][8];
  if (!PRE) {
    vf[0] = vfrag(vb, c, 0);
    vf[1] = vfrag(vb, c, 1);
  }
  if (SOFT) {
    suma = 0.0f;
    read_inv(sb, c, 0, inv[0]);
  }
  step_fence();
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int b = i & 1, db = i >> 1;
    if (ASM)
      pv_mfma8(o[b][db], vf[db & 1], pc[b], one, eb[b]);
    else
      o[b][db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf[db & 1], pc[b], o[b][db], 0, 0, 0, 127, 0, eb[b]);
    if (b == 1 && db + 2 < 4) vf[db & 1] = vfrag(vb, c, db + 2);
    if (SOFT) {
#pragma unroll
      for (int e = 4 * i; e < 4 * i + 4; ++e) exp_step(sb, c, sa, suma, inv, e);
    }
    step_fence();
  }
  if (SOFT) {
    exp_finish(sa, suma, inv);
    asm volatile("" : "+v"(suma));
  }
}

// All 32 exponentials of one block's tile and their sum of P', unpipelined.
__device__ __forceinline__ float exp_all(const char* sb, const Ctx& c, f32x16_t (&s)[2]) {
  float sum = 0.0f, inv[2][8];
  read_inv(sb, c, 0, inv[0]);
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    exp_step(sb, c, s, sum, inv, e);
    if ((e & 7) == 7) step_fence();  // keeps the temporaries few
  }
  exp_finish(s, sum, inv);
  return sum;
}
__device__ __forceinline__ void conv_all(const f32x16_t (&s)[2], v8i32& p, int eb) {
#pragma unroll
  for (int w = 0; w < 8; ++w) conv_word(s, p, w, eb);
}

__device__ __forceinline__ void tile_end() {
  static_assert(VMEM_PER_TILE == 7, "the wait count below leaves one tile's copies in flight");
  asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
  __syncthreads();
}

// One pipelined iteration: X on tile i + 1's K (slot KS), Y on tile i's V (slot VS).
// sc: tile i's scores (A's already exponentiated), sn: tile i + 1's.
template <int KS, int VS>
__device__ __forceinline__ void iteration(const Ctx& c, int i, Stream& st, const bf16x8_t (&qf)[2][8],
                                          f32x16_t (&o)[2][4], f32x16_t (&sc)[2][2], f32x16_t (&sn)[2][2],
                                          v8i32 (&pc)[2], int (&eb)[2], float (&sum)[2], float (&l_part)[2],
                                          const f32x16_t (&negm)[2], int one) {
  static_assert(KS == (VS + 1) % NS, "X reads the slot after Y's");
  v8i32 vf[2];
  phase_x<KS, true, VS>(c, i + 1, qf, negm, sn, sc, pc, eb, sum, vf, [&]() { issue(c, i + NS - 1, st); });
  l_part[0] += sum[0];
  l_part[1] += sum[1];
  phase_y<VS, true, true>(c, i, pc, eb, o, sn[0], sum[0], vf, one);
  tile_end();
}

// Tile i (slot 0) after the pipelined passes: A's codes, B's exponentials and codes, PV.
__device__ __forceinline__ void finish_tile(const Ctx& c, int i, Stream& st, f32x16_t (&o)[2][4],
                                            f32x16_t (&sc)[2][2], v8i32 (&pc)[2], int (&eb)[2], float (&sum)[2],
                                            float (&l_part)[2], int one) {
  issue(c, i + NS - 1, st);
  const char* sb = c.lds;  // slot 0's scale terms: S_RING is in the offsets
  eb[0] = tile_scale(sum[0], c.eb0);
  conv_all(sc[0], pc[0], eb[0]);
  sum[1] = exp_all(sb, c, sc[1]);
  eb[1] = tile_scale(sum[1], c.eb0);
  conv_all(sc[1], pc[1], eb[1]);
  l_part[0] += sum[0];
  l_part[1] += sum[1];
  v8i32 vf[2];
  float unused_sum;
  phase_y<0, false, false, false>(c, i, pc, eb, o, sc[0], unused_sum, vf, one);
  tile_end();
}

// One tile (slot SLOT), unpipelined, with the per-element mask (a no-op for free tiles).
template <int SLOT>
__device__ __forceinline__ void single_tile(const Ctx& c, int i, Stream& st, const bf16x8_t (&qf)[2][8],
                                            f32x16_t (&o)[2][4], f32x16_t (&s)[2][2], v8i32 (&pc)[2], int (&eb)[2],
                                            float (&sum)[2], float (&l_part)[2], const f32x16_t (&negm)[2],
                                            int one) {
  issue(c, i + NS - 1, st);
  f32x16_t unused_s[2][2];
  v8i32 vf[2];
  phase_x<SLOT, false, -2, false, false>(c, i, qf, negm, s, unused_s, pc, eb, sum, vf, []() {});
  const char* sb = c.lds + SLOT * S_TILE;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    mask_tile(s[b], i * BN, c.hi, c.kvis[b]);
    sum[b] = exp_all(sb, c, s[b]);
    eb[b] = tile_scale(sum[b], c.eb0);
    conv_all(s[b], pc[b], eb[b]);
  }
  l_part[0] += sum[0];
  l_part[1] += sum[1];
  float unused_sum;
  phase_y<SLOT, false, false, false>(c, i, pc, eb, o, s[0], unused_sum, vf, one);
  tile_end();
}

}  // namespace d128dual8

__global__ __launch_bounds__(256, 1) void k_attn_f8v_d128_dual(const AttnArgs a) {
  using namespace d128dual8;
  __shared__ __align__(1024) char lds[LDS_BYTES];

  const int n_qt = (a.Lq + BM - 1) / BM;
  const int item = xcd_item(blockIdx.x, n_qt * a.H);  // one head's tiles on one XCD
  const int h = item / n_qt, qt = item - h * n_qt;

  Ctx c;
  c.g.v_mem = static_cast<const char*>(a.v_mem);
  c.g.v_ring = static_cast<const char*>(a.v_ring);
  c.g.v_cur = static_cast<const char*>(a.v_cur);
  c.g.v_ref = static_cast<const char*>(a.v_ref);
  c.g.frame_bytes = (int64_t)a.T * a.H * V8_ROW;
  c.g.T = a.T;
  c.g.Lk = a.Lk;
  c.g.nf = a.Lk / a.T;
  c.g.ref_len = a.hist.ref_len;
  c.g.mem_end = a.hist.ref_len + a.hist.mem_len;
  c.g.nh = a.hist.ref_len + a.hist.mem_len + a.hist.win_len;
  c.g.M = a.hist.M;
  c.g.R = a.hist.R;
  c.g.mem_slot0 = a.hist.mem_slot0;
  c.g.ring_slot0 = a.hist.ring_slot0;
  c.g.s_last = (a.Lk + BN - 1) / BN * BN - 8;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.hi = c.lane >> 5;
  c.lr = c.lane & 31;
  c.lds = lds;
  c.lds_u32 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  c.kbase = static_cast<const char*>(a.k) + (int64_t)h * a.k_head_stride * 2;
  c.hrow = (int64_t)a.H * V8_ROW;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = c.wave * 16 + i * 4 + (c.lane >> 4);
    c.crow[i] = r;
    c.koff[i] = r * ROW_BYTES + ((c.lane & 15) ^ swz(r)) * 16;
  }
  // V copies: lane l moves 16 B of row 16 wave + 8 i + l / 8; its LDS position l mod 8
  // holds the row's chunk (l mod 8) ^ (row mod 8), so the transposed reads (8 consecutive
  // rows, one chunk) hit 8 different 16-byte positions
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = c.wave * 16 + i * 8 + (c.lane >> 3);
    c.vrow[i] = r;
    c.voff[i] = (r * a.H + h) * V8_ROW + ((c.lane & 7) ^ (r & 7)) * 16;
  }
  {
    const int m = perm32(c.lr);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) c.kread[kk] = m * ROW_BYTES + (((2 * kk + c.hi) ^ swz(m)) * 16);
    // V^T reads: 16-lane group g covers channels 16 (g mod 2) of the 32-channel block and
    // keys 8 (g / 2) of each 16-key chunk; lane i addresses row i / 2, byte half i mod 2
    const int g = c.lane >> 4, i = c.lane & 15;
    const int vr = (g >> 1) * 8 + (i >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db)
      c.vread[db] = V_RING + vr * V8_ROW + (((2 * db + (g & 1)) ^ (vr & 7)) * 16) + (i & 1) * 8;
    c.sread = S_RING + c.hi * 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = kb * 32 + m;
      c.lread[kb] = S_RING + (key >> 3) * 64 + 32 + (key & 7) * 4;
    }
  }
  c.vsbase = reinterpret_cast<const char*>(a.vscale + ((c.lane & 15) < 8 ? 1 : 2) * a.vs_plane +
                                           (int64_t)h * a.vs_head_stride + (c.lane & 7));
  {
    float smax = 0.0f;
#pragma unroll
    for (int p = 0; p < kVmaxParts; ++p) smax = fmaxf(smax, a.vmax[h * kVmaxParts + p]);
    // s_v < 2^E_h for every key of the head
    const int eh = (smax > 0.0f && smax < INFINITY) ? __builtin_amdgcn_frexp_expf(smax) : 0;
    c.eb0 = eh - 7;
    const u32x4_t ones = {c.hi ? 0u : 0x3F803F80u, 0u, 0u, 0u};  // bf16 (1, 1, 0, ...)
    c.augb = __builtin_bit_cast(bf16x8_t, ones);
  }
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + (int64_t)h * a.q_head_stride;
  const int q0 = qt * BM;
  int rows[2];
  bf16x8_t qf[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    rows[b] = q0 + c.wave * 64 + b * 32 + c.lr;
    const int rr = rows[b] < a.Lq ? rows[b] : a.Lq - 1;
    c.kvis[b] = a.Lhist + a.block_end[block_of_row(a, rr)];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[b][kk] = in_agprs(rows[b] < a.Lq ? *reinterpret_cast<const bf16x8_t*>(qb + (int64_t)rows[b] * D + kk * 16 + c.hi * 8)
                                          : bf16x8_t{});
  }
  const int last = (q0 + BM < a.Lq ? q0 + BM : a.Lq) - 1;
  const int kend = a.Lhist + a.block_end[block_of_row(a, last)];
  const int kfree = a.Lhist + a.block_end[block_of_row(a, q0)];
  const int nt = (kend + BN - 1) / BN;
  const int n_free = kfree / BN;  // >= 1: every row sees at least the first block's T >= 64 keys
  int one;  // E8M0 1.0, the V operand's block scale, in a VGPR of its own (not rematerialised
            // next to the asm MFMAs that read it)
  asm volatile("v_mov_b32 %0, 127" : "=v"(one));

  f32x16_t o[2][4];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int db = 0; db < 4; ++db) o[b][db] = in_agprs(f32x16_t{});
  float m_ref[2], l_part[2] = {0.0f, 0.0f}, sum[2];
  int eb[2];
  f32x16_t negm[2];
  f32x16_t s0[2][2], s1[2][2];
  v8i32 pc[2] = {v8i32{}, v8i32{}};
  Stream st{0, 0, frame_base(c.g, 0), frame_base(c.g, 1)};
  for (int t = 0; t < NS - 1; ++t) issue(c, t, st);
  asm volatile("s_waitcnt vmcnt(7)" ::: "memory");  // tiles 0 and 1 landed
  __syncthreads();

  // tile 0: scores + log2 s_v from 0; the reference m_ref = the row's largest; A's
  // exponentials
  {
    v8i32 vf[2];
    phase_x<0, false, -2, true, false>(c, 0, qf, negm, s0, s1, pc, eb, sum, vf, []() {});
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float mx = fmaxf(s0[b][0][0], s0[b][1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[b][0][r], s0[b][1][r]));
    m_ref[b] = fmaxf(mx, __shfl_xor(mx, 32)) + (float)MDELTA;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      negm[b][r] = -m_ref[b];
      s0[b][0][r] -= m_ref[b];
      s0[b][1][r] -= m_ref[b];
    }
  }
  sum[0] = exp_all(c.lds, c, s0[0]);

  // Free tiles, pipelined, in passes of four (state in (s0, pc) between passes).
  int i = 0;
  static_assert(NS == 4, "the unrolled loop below walks the slots 0, 1, 2, 3");
  while (i + 4 < n_free) {
    iteration<1, 0>(c, i, st, qf, o, s0, s1, pc, eb, sum, l_part, negm, one);
    iteration<2, 1>(c, i + 1, st, qf, o, s1, s0, pc, eb, sum, l_part, negm, one);
    iteration<3, 2>(c, i + 2, st, qf, o, s0, s1, pc, eb, sum, l_part, negm, one);
    iteration<0, 3>(c, i + 3, st, qf, o, s1, s0, pc, eb, sum, l_part, negm, one);
    i += 4;
  }
  drain_o(o);
  finish_tile(c, i, st, o, s0, pc, eb, sum, l_part, one);
  for (++i; i < nt; ++i) {
    switch (i & 3) {
      case 0: single_tile<0>(c, i, st, qf, o, s0, pc, eb, sum, l_part, negm, one); break;
      case 1: single_tile<1>(c, i, st, qf, o, s0, pc, eb, sum, l_part, negm, one); break;
      case 2: single_tile<2>(c, i, st, qf, o, s0, pc, eb, sum, l_part, negm, one); break;
      default: single_tile<3>(c, i, st, qf, o, s0, pc, eb, sum, l_part, negm, one); break;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the copies issued past the end

  const bool raised = overflow(l_part);
  int bad = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float l = l_part[b] + __shfl_xor(l_part[b], 32);
    const float inv = 1.0f / l;
    bool ok = l > 0.0f && l < 3.0e38f;
    float outv[4][16];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        outv[db][r] = o[b][db][r] * inv;
        ok = ok && (fabsf(outv[db][r]) < 3.0e38f);
      }
    const int row = rows[b];
    if (row < a.Lq) {
      bad |= (ok && !raised) ? 0 : 1;
      uint16_t* ob = static_cast<uint16_t*>(a.out) + ((int64_t)row * a.H + h) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = db * 32 + jg * 8 + c.hi * 4;
          uint2 w2;
          w2.x = pack_bf16x2(outv[db][jg * 4 + 0], outv[db][jg * 4 + 1]);
          w2.y = pack_bf16x2(outv[db][jg * 4 + 2], outv[db][jg * 4 + 3]);
          *reinterpret_cast<uint2*>(ob + d0) = w2;
        }
      if (c.hi == 0 && a.lse) a.lse[(int64_t)h * a.Lq + row] = (m_ref[b] + log2f(l)) * 0.6931471805599453f;
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0 && a.flags) a.flags[item] = bad;
}

// Plain f32 kernel: one lane per query row, 32-key tiles of K and V in LDS.
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(const AttnArgs a) {
  constexpr int BN = 32;
  __shared__ __align__(16) float Ks[BN * D];
  __shared__ __align__(16) float Vs[BN * D];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * 64;
  const int row = q0 + tid;
  const float* qb = static_cast<const float*>(a.q) + (int64_t)h * a.q_head_stride;
  const float* kbase = static_cast<const float*>(a.k) + (int64_t)h * a.k_head_stride;
  float q[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row < a.Lq ? qb[(int64_t)row * D + d] : 0.0f;
    o[d] = 0.0f;
  }
  const int32_t kvis = a.Lhist + a.block_end[block_of_row(a, row < a.Lq ? row : a.Lq - 1)];
  const int32_t last = (q0 + 64 < a.Lq ? q0 + 64 : a.Lq) - 1;
  const int32_t kend = a.Lhist + a.block_end[block_of_row(a, last)];
  float m_run = -INFINITY, l_run = 0.0f;
  for (int k0 = 0; k0 < kend; k0 += BN) {
    __syncthreads();
    for (int c = tid; c < BN * D / 4; c += 64) {
      const int r = c / (D / 4), col = c - r * (D / 4), j = k0 + r;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (j < a.Lk) {
        kv = *reinterpret_cast<const float4*>(kbase + (int64_t)j * D + col * 4);
        int32_t which;
        const int64_t off = v_row_off(a, j, h, &which);
        vv = *reinterpret_cast<const float4*>(v_base<float>(a, which) + off + col * 4);
      }
      *reinterpret_cast<float4*>(&Ks[r * D + col * 4]) = kv;
      *reinterpret_cast<float4*>(&Vs[r * D + col * 4]) = vv;
    }
    __syncthreads();
    float sc[BN];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      float dot = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], Ks[jj * D + d], dot);
      float v = dot;
      if (k0 + jj >= kvis) v = -INFINITY;
      sc[jj] = v;
      mx = fmaxf(mx, v);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
    for (int jj = 0; jj < BN; ++jj) {
      const float p = exp2f(sc[jj] - m_use);
      l_run += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[jj * D + d], o[d]);
    }
    m_run = m_new;
  }
  if (row < a.Lq) {
    const float inv = 1.0f / l_run;
    float* ob = static_cast<float*>(a.out) + ((int64_t)row * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) ob[d] = o[d] * inv;
    if (a.lse) a.lse[(int64_t)h * a.Lq + row] = (m_run + log2f(l_run)) * 0.6931471805599453f;
  }
}

hipError_t launch_attention(const AttnArgs& a, int32_t op_dtype, hipStream_t s) {
  if (a.Lq <= 0) return hipSuccess;
  if (op_dtype == DT_BF16) {
    dim3 grid((a.Lq + 127) / 128, a.H);
    if (a.D == 128 && a.T >= d128dual::BN && a.flags) {
      static_assert(d128dual::BM == d128dual8::BM && d128dual::BN == d128dual8::BN, "one item layout");
      const int items = ((a.Lq + d128dual::BM - 1) / d128dual::BM) * a.H;
      if (a.v_fp8) {
        hipLaunchKernelGGL(k_attn_f8v_d128_dual, dim3(items), dim3(64 * d128dual8::WAVES), 0, s, a);
      } else {
        hipLaunchKernelGGL(k_attn_bf16_d128_dual, dim3(items), dim3(64 * d128dual::WAVES), 0, s, a);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (a.v_fp8)  // flagged tiles only
        hipLaunchKernelGGL((k_attn_bf16<128, true>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((k_attn_bf16<128, false>), grid, dim3(256), 0, s, a);
    } else {
      AttnArgs g = a;
      g.flags = nullptr;
      if (a.D == 128) {
        if (a.v_fp8)
          hipLaunchKernelGGL((k_attn_bf16<128, true>), grid, dim3(256), 0, s, g);
        else
          hipLaunchKernelGGL((k_attn_bf16<128, false>), grid, dim3(256), 0, s, g);
      } else {
        if (a.v_fp8)
          hipLaunchKernelGGL((k_attn_bf16<64, true>), grid, dim3(256), 0, s, g);
        else
          hipLaunchKernelGGL((k_attn_bf16<64, false>), grid, dim3(256), 0, s, g);
      }
    }
  } else if (op_dtype == DT_F32) {
    dim3 grid((a.Lq + 63) / 64, a.H);
    if (a.D == 128)
      hipLaunchKernelGGL(k_attn_f32<128>, grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL(k_attn_f32<64>, grid, dim3(64), 0, s, a);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace lact
