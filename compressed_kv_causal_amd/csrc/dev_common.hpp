// dev_common.hpp -- device helpers: bf16 and OCP e4m3 codecs, vector loads, reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace lact {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest, ties to even; overflow goes to +-inf as IEEE rounding does; NaN stays
// a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP E4M3FN (bias 7, no infinities, S.1111.111 = NaN, largest finite 448, subnormals
// m * 2^-9) through gfx950's conversion instructions, which use this format.
// Decode: exact for every code (NaN codes give NaN).  Encode: round to nearest, ties to
// even mantissa; the value is clamped to [-448, 448] first, so larger magnitudes saturate
// to +-448 (a NaN input gives an unspecified code: the row quantiser only sees finite
// values for finite inputs).  Both agree with the format's definition for every finite
// f32 input and every code (checked exhaustively on the device).

// the four codes of w -> x[0..3] (byte i -> x[i])
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* x) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  x[0] = lo[0];
  x[1] = lo[1];
  x[2] = hi[0];
  x[3] = hi[1];
}

// codes of y[0..3] packed as bytes 0..3
__device__ __forceinline__ uint32_t f32x4_to_e4m3(const float* y) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(y[i], -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

// Row quantiser of the FP8 cache, per (token, head): scale = amax / 448, y = x * (448 / amax)
// (one f32 rounding each; amax = 0 -> scale 1, y = x).
struct RowQuant {
  float scale, inv;
};
__device__ __forceinline__ RowQuant row_quant(float amax) {
  RowQuant q;
  if (amax > 0.0f) {
    q.scale = __fdiv_rn(amax, 448.0f);
    q.inv = __fdiv_rn(448.0f, amax);
  } else {
    q.scale = 1.0f;
    q.inv = 1.0f;
  }
  return q;
}

// max over groups of `width` consecutive lanes (width a power of two <= 64)
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, width));
  return v;
}

// 8 consecutive elements as f32, from f32 / bf16 / fp8(code*scale) storage.
__device__ __forceinline__ void load8_f32(const float* p, float* x) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8_bf16(const uint16_t* p, float* x) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8_fp8(const uint8_t* p, float scale, float* x) {
  uint2 v = *reinterpret_cast<const uint2*>(p);
  e4m3x4_to_f32(v.x, x);
  e4m3x4_to_f32(v.y, x + 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= scale;
}

__device__ __forceinline__ void store8_f32(float* p, const float* x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
// Two values rounded to bf16 (nearest, ties to even; one v_cvt_pk_bf16_f32), lo in the low
// half.  Finite values round exactly as f32_to_bf16; a NaN stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void store8_bf16(uint16_t* p, const float* x) {
  uint4 v;
  v.x = pack_bf16x2(x[0], x[1]);
  v.y = pack_bf16x2(x[2], x[3]);
  v.z = pack_bf16x2(x[4], x[5]);
  v.w = pack_bf16x2(x[6], x[7]);
  *reinterpret_cast<uint4*>(p) = v;
}
// quantises 8 values with the row's inverse scale and stores 8 codes
__device__ __forceinline__ void store8_fp8(uint8_t* p, const float* x, float inv) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * inv;
  *reinterpret_cast<uint2*>(p) = make_uint2(f32x4_to_e4m3(y), f32x4_to_e4m3(y + 4));
}

// Load 8 input elements (q dtype: F32 or BF16) starting at element offset off.
__device__ __forceinline__ void load8_in(const void* base, int32_t dtype, int64_t off, float* x) {
  if (dtype == DT_F32)
    load8_f32(static_cast<const float*>(base) + off, x);
  else
    load8_bf16(static_cast<const uint16_t*>(base) + off, x);
}

// Load 8 stored elements (kv dtype) at element offset off; row_scale used for FP8.
__device__ __forceinline__ void load8_kv(const void* base, int32_t dtype, int64_t off,
                                         float row_scale, float* x) {
  if (dtype == DT_F32)
    load8_f32(static_cast<const float*>(base) + off, x);
  else if (dtype == DT_BF16)
    load8_bf16(static_cast<const uint16_t*>(base) + off, x);
  else
    load8_fp8(static_cast<const uint8_t*>(base) + off, row_scale, x);
}

// Store 8 elements in an operand dtype (F32 or BF16) at element offset off.
__device__ __forceinline__ void store8_op(void* base, int32_t dtype, int64_t off, const float* x) {
  if (dtype == DT_F32)
    store8_f32(static_cast<float*>(base) + off, x);
  else
    store8_bf16(static_cast<uint16_t*>(base) + off, x);
}

// Store 8 elements in dtype at element offset off.  FP8 quantises the row: every lane of
// the row's group (lanes_per_row consecutive lanes) must call this together; the row's
// scale is returned (and written by the caller).
template <int lanes_per_row>
__device__ __forceinline__ float store8_kv(void* base, int32_t dtype, int64_t off, const float* x) {
  if (dtype == DT_F32) {
    store8_f32(static_cast<float*>(base) + off, x);
    return 1.0f;
  }
  if (dtype == DT_BF16) {
    store8_bf16(static_cast<uint16_t*>(base) + off, x);
    return 1.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = group_max<lanes_per_row>(amax);
  RowQuant rq = row_quant(amax);
  store8_fp8(static_cast<uint8_t*>(base) + off, x, rq.inv);
  return rq.scale;
}

// Workgroup b of a launch runs on XCD b mod 8, and each XCD has its own L2.  Maps the
// workgroup's linear id b to an item of [0, n) so that each XCD takes one contiguous range
// of items: neighbouring items, which share cache lines, then share one L2.  A bijection
// on [0, n).
__device__ __forceinline__ int32_t xcd_item(int32_t b, int32_t n) {
  const int32_t x = b & 7, j = b >> 3;
  const int32_t q8 = n >> 3, r8 = n & 7;
  return x < r8 ? x * (q8 + 1) + j : r8 * (q8 + 1) + (x - r8) * q8 + j;
}

// Sources of a key frame's rows.
enum : int32_t { SRC_RING = 0, SRC_MEM = 1, SRC_CUR = 2, SRC_REF = 3 };

// Storage of history key frame fi: SRC_REF, SRC_MEM or SRC_RING, and its slot there.
__device__ __forceinline__ int32_t hist_src(const HistMap& m, int32_t fi, int32_t* slot) {
  if (fi < m.ref_len) {
    *slot = fi;
    return SRC_REF;
  }
  fi -= m.ref_len;
  int32_t s;
  if (fi < m.mem_len) {
    s = m.mem_slot0 + fi;
    *slot = s >= m.M ? s - m.M : s;
    return SRC_MEM;
  }
  s = m.ring_slot0 + (fi - m.mem_len);
  *slot = s >= m.R ? s - m.R : s;
  return SRC_RING;
}

}  // namespace lact
