// k_attn.hip -- block attention over [reference | memory | window | current] on gfx950.
//
// O = softmax(Q K^T / sqrt(D) + mask) V per head (walkthrough "SoulX-LiveAct", section
// "ConvKV Memory": context = long-term memory, short-term window, current block; section
// "Neighbor Forcing": block-wise causal mask of block size m).  Memory and window keys are
// visible to every query; current key j is visible to query i iff block(j) <= block(i), so
// query row i sees exactly the key prefix [0, Lhist + block_end[block(i)]).
//
// Kernels:
//   k_attn_bf16_d128  the D = 128 production kernel (described at its definition).
//   k_attn_bf16<D>    exact online-softmax flash attention on v_mfma_f32_32x32x16_bf16,
//                     4 waves x 32 query rows, 64-key tiles staged in LDS (K row-major, V
//                     transposed by the staging threads), running max with rescaling: the
//                     kernel for D = 64 and T < 64, and the exact fallback of the D = 128
//                     kernel for the query tiles it flags.
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

template <int D>
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
        if (j < a.Lk) {
          int32_t which;
          const int64_t off = v_row_off(a, j, h, &which);
          vv[t] = *reinterpret_cast<const uint4*>(v_base<uint16_t>(a, which) + off + dchunk * 8);
        }
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
// k_attn_bf16_d128: the D = 128 production kernel (T >= 64).
//
//   * 256 query rows per workgroup, 8 waves x 32 rows: two waves per SIMD, so one wave's
//     softmax (VALU) and barrier waits overlap the other's MFMAs.
//   * Key tiles of BN = 64 rows are copied global -> LDS with global_load_lds (16 B per
//     lane, no registers) into a ring of NS = 4 stages: tile j + 3 is in flight while tile
//     j is computed.  Rows are stored with an XOR swizzle of their 16-byte chunks:
//         chunk c of key row r sits at position c ^ swz(r), swz(r) = ((r & 3) << 2) | ((r >> 2) & 3)
//     swz is a bijection over 16 consecutive rows (K fragment reads, ds_read_b128 of 16 rows
//     x one chunk, hit 16 distinct 16-byte slots) and puts the low row bits above the chunk
//     bits (a V^T fragment read, ds_read_b64_tr_b16 of 4 rows x 4 chunks per 32 lanes, hits
//     16 distinct slots), so neither read has bank conflicts.
//   * V^T fragments come from the transposing LDS read: within each 16-lane group, lanes
//     4t..4t+3 address key row t (16 consecutive channels) and lane i receives channel i
//     of rows 0..3 -- the consecutive keys of one channel the MFMA A operand needs.
//   * Addressing costs almost no VALU work per tile.  Copies: the tile's first key frame
//     and token and the V bases of that frame and the next (memory slot, raw ring slot or
//     staged block frame) are scalar state; a lane adds its constant row offset to one of
//     the two (a 64-key tile spans at most two frames since T >= 64).  Fragment reads: the
//     per-lane LDS offsets of all K and V^T fragments are loop invariants; the ring slot
//     and the fragment's key block or chunk are the instruction's immediate offset, with
//     the unmasked tile loop unrolled by NS so the slot is a compile-time constant.
//   * Softmax with a lazily raised reference: m = the row's max over the first key tile.
//     The staged queries carry log2(e)/sqrt(D), and every QK^T MFMA chain starts from the
//     broadcast -m instead of 0, so the chain's output q.k - m is already the base-2
//     exponent of the probability: the softmax spends one v_exp per score and nothing
//     else.  There is no running max and no per-tile rescale of O; since m never exceeds
//     the true row max, terms are
//     only ever too large, never lost.  Only when a lane's tile sum reaches 2^64 (scores
//     far above m, e.g. from outlier channels) does the wave raise m by a power of two and
//     scale O and l exactly (see tile()).  If l or O still ends up not finite, the
//     workgroup marks itself in `flags` and the exact online-softmax kernel redoes its rows.
//   * Workgroup -> (head, query tile) mapping keeps each XCD (every 8th workgroup id) on
//     the tiles of one head at a time, so that head's K/V stream once through one L2.
// ---------------------------------------------------------------------------------------
namespace d128 {

constexpr int D = 128, BM = 256, BN = 64, NS = 4, WAVES = 8;
constexpr int ROW_BYTES = D * 2;
constexpr int TILE_BYTES = BN * ROW_BYTES;  // 16 KiB
constexpr int V_RING = NS * TILE_BYTES;     // V slots follow the K slots in LDS
constexpr int VMEM_PER_TILE = 4;            // copy instructions per wave per tile (K 2, V 2)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// One 1 KiB global -> LDS copy per wave (16 B per lane, lane l lands at LDS address
// m0 + 16 l; m0 is wave-uniform).  Issued through inline asm: the compiler then does not
// treat it as an LDS write it must wait for before every later LDS read (it would insert
// vmcnt(0) right after the copy and the prefetch would never overlap); the ring's own
// "s_waitcnt vmcnt + barrier" orders the copies with the reads.  No VGPR is written.
__device__ __forceinline__ void copy_to_lds(const void* src, unsigned m0) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0) : "memory");
}

// The scalars the copies need, as plain values (the kernel's argument block stays in the
// constant kernarg segment: taking a field by a computed offset would make the compiler
// copy the whole block into scratch memory and every use of it per-lane).
struct Geo {
  const char* v_mem;
  const char* v_ring;
  const char* v_cur;
  const char* v_ref;
  int64_t frame_bytes;  // one V frame, T * H * D * 2
  int T, Lk, nf, ref_len, mem_end, nh, M, R, mem_slot0, ring_slot0;
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

struct Ctx {
  Geo g;
  const char* kbase;  // this head's rotated keys [Lk][128]
  char* lds;
  unsigned lds_u32;   // LDS address of the ring (for M0)
  int h, wave, lane, hi, lr, kvis;
  int64_t hrow;       // bytes between consecutive tokens of one V frame (H * D * 2)
  // copies: the two 4-row groups of a tile this lane copies
  int crow[2];        // row inside the tile
  int koff[2];        // crow * 256 + chunk * 16 (bytes from the tile's first K row)
  int voff[2];        // (crow * H + h) * 256 + chunk * 16 (bytes from the V row of token 0)
  // fragment reads: LDS byte offsets from the ring base (slot 0)
  int kread[8];       // K fragment kk of key block 0 (+ 8 KiB for block 1)
  int vread[4][2];    // the two transposed reads of V^T fragment db, chunk 0 (+ 4 KiB per chunk)
};

// Scalar stream state of the copies: frame and token of the first key of the next tile,
// and the V bases of that frame and the next (recomputed when a tile crosses a frame).
struct Stream {
  int f0, u0;
  const char* baseA;
  const char* baseB;
};

// Copy tile t's 64 key rows of K and V into ring slot t % NS, then advance the stream.
__device__ __forceinline__ void issue(const Ctx& c, int t, Stream& st) {
  const Geo& a = c.g;
  const unsigned slot = (unsigned)(t % NS);
  const unsigned kdst = c.lds_u32 + slot * TILE_BYTES + (unsigned)c.wave * 8 * ROW_BYTES;
  const unsigned vdst = kdst + V_RING;
  if ((t + 1) * BN <= a.Lk) {
    const char* ktile = c.kbase + (int64_t)t * TILE_BYTES;
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_to_lds(ktile + c.koff[i], kdst + i * 4 * ROW_BYTES);
  } else {  // rows past the last key repeat it
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int key = t * BN + c.crow[i];
      key = key < a.Lk ? key : a.Lk - 1;
      copy_to_lds(c.kbase + (int64_t)key * ROW_BYTES + (c.koff[i] & (ROW_BYTES - 1)), kdst + i * 4 * ROW_BYTES);
    }
  }
  const char* vA = st.baseA + st.u0 * c.hrow;
  if (st.u0 + BN <= a.T) {  // the whole tile lies in frame f0
#pragma unroll
    for (int i = 0; i < 2; ++i) copy_to_lds(vA + c.voff[i], vdst + i * 4 * ROW_BYTES);
  } else {
    const char* vB = st.baseB + (st.u0 - a.T) * c.hrow;
#pragma unroll
    for (int i = 0; i < 2; ++i)
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

// LDS address helpers: SLOT >= 0 is a compile-time ring slot, SLOT < 0 takes tile j's.
template <int SLOT>
__device__ __forceinline__ int slot_of(int j) { return SLOT >= 0 ? SLOT : j % NS; }

template <bool MASK>
__device__ __forceinline__ void mask_block(f32x16_t& s, int key0, int hi, int kvis) {
  if (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + perm32(((r >> 2) << 3) + (hi << 2) + (r & 3));
      if (key >= kvis) s[r] = -INFINITY;
    }
  }
}

// Scheduling fence between pipeline steps (no instruction crosses it): without it the
// compiler moves each MFMA up next to its fragment read and reuses one fragment register,
// exposing the full LDS latency on every MFMA.
__device__ __forceinline__ void step_fence() { __builtin_amdgcn_sched_barrier(0); }

// S^T of one 64-key tile (two 32-key blocks) from the K rows in LDS, masked, on top of
// `init` (the broadcast -m_ref of the lane's row: the chains then produce the exponents
// of the probabilities directly).  The two key blocks are independent MFMA chains,
// interleaved; K fragments are read three steps ahead of their MFMAs.
template <bool MASK, int SLOT>
__device__ __forceinline__ void qk_tile(const Ctx& c, int j, const bf16x8_t (&qf)[8], const f32x16_t& init,
                                        f32x16_t (&s)[2]) {
  const char* kb = c.lds + slot_of<SLOT>(j) * TILE_BYTES;
  auto kfrag = [&](int kk, int kb2) {
    return *reinterpret_cast<const bf16x8_t*>(kb + c.kread[kk] + kb2 * 32 * ROW_BYTES);
  };
  constexpr int AHEAD = 3;  // steps of two MFMAs (64 cycles) between a read and its use
  bf16x8_t kf[AHEAD + 1][2];
#pragma unroll
  for (int kk = 0; kk < AHEAD; ++kk) {
    kf[kk][0] = kfrag(kk, 0);
    kf[kk][1] = kfrag(kk, 1);
  }
  step_fence();
  s[0] = init;
  s[1] = init;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    if (kk + AHEAD < 8) {
      kf[(kk + AHEAD) % (AHEAD + 1)][0] = kfrag(kk + AHEAD, 0);
      kf[(kk + AHEAD) % (AHEAD + 1)][1] = kfrag(kk + AHEAD, 1);
    }
    s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % (AHEAD + 1)][0], qf[kk], s[0], 0, 0, 0);
    s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % (AHEAD + 1)][1], qf[kk], s[1], 0, 0, 0);
    step_fence();
  }
  mask_block<MASK>(s[0], j * BN, c.hi, c.kvis);
  mask_block<MASK>(s[1], j * BN + 32, c.hi, c.kvis);
}

// V^T fragment (16 keys of chunk ch, channels 32 db .. 32 db + 31).
__device__ __forceinline__ bf16x8_t vfrag(const char* vb, const Ctx& c, int ch, int db) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + c.vread[db][0] + ch * 16 * ROW_BYTES));
  const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vb + c.vread[db][1] + ch * 16 * ROW_BYTES));
  bf16x8_t vf;
  __builtin_memcpy(&vf, &lo, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&vf) + 8, &up, 8);
  return vf;
}

// p = exp2(s - sub) in place (sub = 0 when s already holds the exponents); returns this
// lane's sum of the 32 probabilities.
template <bool SUB>
__device__ __forceinline__ float exp_tile(f32x16_t (&s)[2], float sub) {
  float sum = 0.0f;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(SUB ? s[kb2][r] - sub : s[kb2][r]);
      s[kb2][r] = e;
      sum += e;
    }
  return sum;
}

// Tile j: issue the copy of tile j + NS - 1 into the slot tile j - 1 used (every wave was
// done with it before the last barrier), compute tile j, then wait until tile j + 1 has
// landed (the copies of tiles j + 2 .. j + NS - 1 stay in flight) and sync.  Tiles past
// the end are copied too (clamped rows, harmless), so the wait count is a constant.
//
// Reference raise: a lane sum of 2^64 or more means a row met scores far above its
// reference.  The wave then takes each such row's largest probability of the tile, 2^e *
// [1, 2), and divides that row's probabilities, O and l by 2^e (exact power-of-two scaling)
// while m_ref moves up by e.  Ordinary data never takes this branch; scores with large
// outliers take it a few times per row at most.  A probability that is already infinite
// (a score >= 128 above the reference) cannot be rescaled: l and O become infinite and the
// workgroup hands its rows to the exact pass.
template <bool MASK, bool FIRST, int SLOT>
__device__ __forceinline__ void tile(const Ctx& c, int j, const bf16x8_t (&qf)[8], f32x16_t (&o)[4],
                                     float& m_ref, f32x16_t& negm, float& l_part, Stream& st) {
  const char* vb = c.lds + slot_of<SLOT>(j) * TILE_BYTES;  // + vread (which holds V_RING)
  issue(c, j + NS - 1, st);
  f32x16_t s[2];
  qk_tile<MASK, SLOT>(c, j, qf, negm, s);  // tile 0: negm = 0
  float sum;
  if (FIRST) {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    m_ref = fmaxf(mx, __shfl_xor(mx, 32));
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
    sum = exp_tile<true>(s, m_ref);
  } else {
    sum = exp_tile<false>(s, 0.0f);
  }
  if (!FIRST && __builtin_expect(__any(!(sum < 0x1p64f)), 0)) {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // e = floor(log2(mx)) for a finite mx >= 2, else 0
    const int e = (mx >= 2.0f && mx < INFINITY) ? __builtin_amdgcn_frexp_expf(mx) - 1 : 0;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb2][r] = __builtin_ldexpf(s[kb2][r], -e);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = __builtin_ldexpf(o[db][r], -e);
    l_part = __builtin_ldexpf(l_part, -e);
    sum = __builtin_ldexpf(sum, -e);
    m_ref += (float)e;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
  }
  l_part += sum;
  bf16x8_t p[4];
#pragma unroll
  for (int ch = 0; ch < 4; ++ch)
#pragma unroll
    for (int t = 0; t < 8; ++t) p[ch][t] = (__bf16)s[ch >> 1][8 * (ch & 1) + t];
  // O^T += V^T P^T: 16 MFMAs (chunk ch, channel block db) in 4 independent chains, V^T
  // fragments read four MFMAs (128 cycles) ahead
  constexpr int VAHEAD = 4;
  bf16x8_t vf[VAHEAD + 1];
#pragma unroll
  for (int i = 0; i < VAHEAD; ++i) vf[i] = vfrag(vb, c, i >> 2, i & 3);
  step_fence();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i + VAHEAD < 16) vf[(i + VAHEAD) % (VAHEAD + 1)] = vfrag(vb, c, (i + VAHEAD) >> 2, (i + VAHEAD) & 3);
    o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % (VAHEAD + 1)], p[i >> 2], o[i & 3], 0, 0, 0);
    step_fence();
  }
  static_assert((NS - 2) * VMEM_PER_TILE == 8, "the wait count below assumes 4 stages");
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  __syncthreads();
}

}  // namespace d128

__global__ __launch_bounds__(512, 1) void k_attn_bf16_d128(const AttnArgs a) {
  using namespace d128;
  __shared__ __align__(1024) char lds[2 * NS * TILE_BYTES];

  // XCD-aware mapping: workgroup id b runs on XCD b % 8; give each XCD a contiguous range
  // of (head, query tile) items so one head's tiles run on one XCD together.
  const int n_qt = (a.Lq + BM - 1) / BM;
  const int total = n_qt * a.H;
  const int b = blockIdx.x;
  const int x = b & 7, jx = b >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int item = x < r8 ? x * (q8 + 1) + jx : r8 * (q8 + 1) + (x - r8) * q8 + jx;
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
  c.h = h;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.lane = threadIdx.x & 63;
  c.hi = c.lane >> 5;
  c.lr = c.lane & 31;
  c.lds = lds;
  c.lds_u32 = (unsigned)(uintptr_t)(__attribute__((address_space(3))) char*)lds;
  c.kbase = static_cast<const char*>(a.k) + (int64_t)h * a.k_head_stride * 2;
  c.hrow = (int64_t)a.H * ROW_BYTES;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = c.wave * 8 + i * 4 + (c.lane >> 4);
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

  const int row = q0 + c.wave * 32 + c.lr;
  const int rr = row < a.Lq ? row : a.Lq - 1;
  c.kvis = a.Lhist + a.block_end[block_of_row(a, rr)];
  bf16x8_t qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = row < a.Lq ? *reinterpret_cast<const bf16x8_t*>(qb + (int64_t)row * D + kk * 16 + c.hi * 8)
                        : bf16x8_t{};
  const int last = (q0 + BM < a.Lq ? q0 + BM : a.Lq) - 1;
  const int kend = a.Lhist + a.block_end[block_of_row(a, last)];
  const int kfree = a.Lhist + a.block_end[block_of_row(a, q0)];
  const int nt = (kend + BN - 1) / BN;
  const int n_free = kfree / BN;  // tiles every row of the workgroup sees completely

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};
  float m_ref = 0.0f, l_part = 0.0f;
  f32x16_t negm = f32x16_t{};  // -m_ref in every element (the QK^T chains' starting value)
  Stream st{0, 0, frame_base(c.g, 0), frame_base(c.g, 1)};
  for (int t = 0; t < NS - 1; ++t) issue(c, t, st);
  asm volatile("s_waitcnt vmcnt(8)" ::: "memory");  // tile 0 landed
  __syncthreads();

  if (n_free > 0)
    tile<false, true, 0>(c, 0, qf, o, m_ref, negm, l_part, st);
  else
    tile<true, true, 0>(c, 0, qf, o, m_ref, negm, l_part, st);
  int j = 1;
  const int free_end = n_free < nt ? n_free : nt;
  static_assert(NS == 4, "the unrolled loop below walks the slots 1, 2, 3, 0");
  for (; j + 4 <= free_end; j += 4) {
    tile<false, false, 1>(c, j, qf, o, m_ref, negm, l_part, st);
    tile<false, false, 2>(c, j + 1, qf, o, m_ref, negm, l_part, st);
    tile<false, false, 3>(c, j + 2, qf, o, m_ref, negm, l_part, st);
    tile<false, false, 0>(c, j + 3, qf, o, m_ref, negm, l_part, st);
  }
  for (; j < free_end; ++j) tile<false, false, -1>(c, j, qf, o, m_ref, negm, l_part, st);
  for (; j < nt; ++j) tile<true, false, -1>(c, j, qf, o, m_ref, negm, l_part, st);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the copies issued past the end

  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l;
  bool ok = l > 0.0f && l < 3.0e38f;
  float outv[4][16];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      outv[db][r] = o[db][r] * inv;
      ok = ok && (fabsf(outv[db][r]) < 3.0e38f);
    }
  int bad = 0;
  if (row < a.Lq) {
    bad = ok ? 0 : 1;
    uint16_t* ob = static_cast<uint16_t*>(a.out) + ((int64_t)row * a.H + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int d0 = db * 32 + jg * 8 + c.hi * 4;
        uint2 w2;
        w2.x = (uint32_t)f32_to_bf16(outv[db][jg * 4 + 0]) | ((uint32_t)f32_to_bf16(outv[db][jg * 4 + 1]) << 16);
        w2.y = (uint32_t)f32_to_bf16(outv[db][jg * 4 + 2]) | ((uint32_t)f32_to_bf16(outv[db][jg * 4 + 3]) << 16);
        *reinterpret_cast<uint2*>(ob + d0) = w2;
      }
    if (c.hi == 0 && a.lse) a.lse[(int64_t)h * a.Lq + row] = (m_ref + log2f(l)) * 0.6931471805599453f;
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
    if (a.D == 128 && a.T >= d128::BN && a.flags) {
      const int items = ((a.Lq + d128::BM - 1) / d128::BM) * a.H;
      hipLaunchKernelGGL(k_attn_bf16_d128, dim3(items), dim3(64 * d128::WAVES), 0, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(256), 0, s, a);  // flagged tiles only
    } else {
      AttnArgs g = a;
      g.flags = nullptr;
      if (a.D == 128)
        hipLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(256), 0, s, g);
      else
        hipLaunchKernelGGL(k_attn_bf16<64>, grid, dim3(256), 0, s, g);
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
