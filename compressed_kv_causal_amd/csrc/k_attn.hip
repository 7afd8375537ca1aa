// k_attn.hip -- block attention over [memory | window | current] on gfx950.
//
// O = softmax(Q K^T / sqrt(D) + mask) V per head (walkthrough "SoulX-LiveAct", section
// "ConvKV Memory": context = long-term memory, short-term window, current block; section
// "Neighbor Forcing": block-wise causal mask of block size m).  Memory and window keys are
// visible to every query; current key j is visible to query i iff block(j) <= block(i), so
// query row i sees exactly the key prefix [0, Lhist + block_end[block(i)]).
//
// Kernels:
//   k_attn_bf16<D>  flash attention on v_mfma_f32_32x32x16_bf16, 4 waves x 32 query rows,
//                   64-key tiles staged in LDS (K row-major, V transposed), online softmax
//                   in the exp2 domain, tiles past the block-causal prefix never visited.
//   k_attn_f32<D>   plain f32 FMA kernel (one lane per query row) for the f32 cache.
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

// Element offset of V row (key j, head h).  Key frame fi = j / T of [memory | window |
// current]: memory and window frames are read where they are stored (raw ring or memory
// slot), the block's frames from the staged copy.
__device__ __forceinline__ int64_t v_row_off(const AttnArgs& a, int32_t j, int32_t h,
                                             int32_t* which) {
  const int32_t fi = j / a.T;
  const int32_t u = j - fi * a.T;
  const int32_t nh = a.hist.mem_len + a.hist.win_len;
  int32_t slot;
  if (fi < nh) {
    slot = hist_slot(a.hist, fi);
    *which = fi < a.hist.mem_len ? 1 : 0;
  } else {
    slot = fi - nh;
    *which = 2;
  }
  return (((int64_t)slot * a.T + u) * a.H + h) * a.D;
}

template <typename T>
__device__ __forceinline__ const T* v_base(const AttnArgs& a, int32_t which) {
  return static_cast<const T*>(which == 1 ? a.v_mem : (which == 0 ? a.v_ring : a.v_cur));
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
        float v = s[kb][j] * a.scale_log2;
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
      float v = dot * a.scale_log2;
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

hipError_t launch_attention(const AttnArgs& a, int32_t kv_dtype, hipStream_t s) {
  if (a.Lq <= 0) return hipSuccess;
  if (kv_dtype == DT_BF16) {
    dim3 grid((a.Lq + 127) / 128, a.H);
    if (a.D == 128)
      hipLaunchKernelGGL(k_attn_bf16<128>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(k_attn_bf16<64>, grid, dim3(256), 0, s, a);
  } else if (kv_dtype == DT_F32) {
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
