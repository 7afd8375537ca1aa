// mb.hip -- measurement kernels for bench.py: what one MI355X (gfx950) sustains on the
// patterns the step's kernels use, so each of them can be read against a measured
// ceiling beside the published peaks.  Not part of the method's path.
//
//   mb_mfma_loop   back-to-back matrix-core instructions, 4 independent accumulator
//                  chains per wave, 2 waves per SIMD: v_mfma_f32_32x32x16_bf16 or
//                  v_mfma_f32_32x32x64_f8f6f4
//   mb_copy        streaming copy, two 16 B elements per lane, one pass (1:1 read:write)
//   mb_copy5       5 streams in, 1 out, element-wise sum (the compressor's 5:1 mix)
//   mb_read        read-only stream (1:0)
//   mb_mfma_lds    the bf16 MFMA stream with each A operand read from LDS (1 KiB per MFMA):
//                  one ds_read_b128 per lane, or two transposing ds_read_b64_tr_b16 per lane
//                  (the attention kernel's K and V^T fragment reads)
//   mb_overlap     a bf16 MFMA stream and a stream of exponentials with their running sums
//                  (the softmax's work), alone, in two waves of one SIMD, or interleaved in
//                  one wave
#include <hip/hip_runtime.h>

#include <cstdint>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int v8i32 __attribute__((ext_vector_type(8)));

template <bool FP8>
__global__ __launch_bounds__(512) void k_mfma_loop(const float* seed, float* sink, int iters) {
  f32x16_t acc[4] = {};
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
  v8i32 a8, b8;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)seed[(lane + i) & 63];
    b[i] = (__bf16)seed[(lane + 3 * i) & 63];
    a8[i] = 0x38383838 + i;   // small e4m3 values
    b8[i] = 0x30303030 + i;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (FP8)
        acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[m], 0, 0, 0, 0, 0, 0);
      else
        acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[m][j];
  if (s == 1234.5f) sink[blockIdx.x] = s;   // keeps the loop alive; never true in practice
}

// n16: number of 16-byte elements.  One pass: lane i of the grid moves elements i and
// i + half (both loads issued before either store), a grid of n16 / 512 workgroups --
// the shape of the step's own streaming kernels (one row chunk per lane, no loop).
__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                              int64_t n16) {
  const int64_t half = (n16 + 1) / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= half) return;
  const bool two = i + half < n16;
  const uint4 a = src[i];
  uint4 b = make_uint4(0, 0, 0, 0);
  if (two) b = src[i + half];
  dst[i] = a;
  if (two) dst[i + half] = b;
}

// five inputs, one output, element-wise sum; one element per lane
__global__ __launch_bounds__(256) void k_copy5(const uint4* __restrict__ s0, const uint4* __restrict__ s1,
                                               const uint4* __restrict__ s2, const uint4* __restrict__ s3,
                                               const uint4* __restrict__ s4, uint4* __restrict__ dst,
                                               int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const uint4 a = s0[i], b = s1[i], c = s2[i], d = s3[i], e = s4[i];
  dst[i] = make_uint4(a.x + b.x + c.x + d.x + e.x, a.y + b.y + c.y + d.y + e.y,
                      a.z + b.z + c.z + d.z + e.z, a.w + b.w + c.w + d.w + e.w);
}

// read-only stream: two elements per lane, the XOR of everything kept in one word per
// workgroup
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ src, uint32_t* sink,
                                              int64_t n16) {
  const int64_t half = (n16 + 1) / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t x = 0;
  if (i < half) {
    const uint4 a = src[i];
    x = a.x ^ a.y ^ a.z ^ a.w;
    if (i + half < n16) {
      const uint4 b = src[i + half];
      x ^= b.x ^ b.y ^ b.z ^ b.w;
    }
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x & 1023] = x;   // keeps the loads; data never matches
}

// MFMAs fed from LDS: 8 waves (2 per SIMD), every wave reads the 16 KiB buffer as 16
// fragments of 1 KiB per pass, each fragment read 4 MFMAs before its MFMA.  TR = 0: one
// 16 B ds_read_b128 per lane; TR = 1: two 8 B ds_read_b64_tr_b16 per lane.  All reads stay
// inside the buffer (fragment f covers bytes [1024 f, 1024 f + 1024)).
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <bool TR>
__device__ __forceinline__ bf16x8_t lds_frag(const char* buf, int f, int lane) {
  if (TR) {
    const char* b = buf + f * 1024 + lane * 8;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)b);
    const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(b + 512));
    bf16x8_t v;
    __builtin_memcpy(&v, &lo, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&v) + 8, &up, 8);
    return v;
  }
  return *reinterpret_cast<const bf16x8_t*>(buf + f * 1024 + lane * 16);
}

template <bool TR>
__global__ __launch_bounds__(512) void k_mfma_lds(const float* seed, float* sink, int iters) {
  __shared__ __align__(16) char buf[16384];
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 16384 / 2; i += 512)
    reinterpret_cast<__bf16*>(buf)[i] = (__bf16)seed[i & 63];
  __syncthreads();
  bf16x8_t b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (__bf16)seed[(lane + 3 * i) & 63];
  f32x16_t acc[4] = {};
  constexpr int AH = 4;
  for (int it = 0; it < iters; ++it) {
    bf16x8_t fr[AH + 1];
#pragma unroll
    for (int f = 0; f < AH; ++f) fr[f] = lds_frag<TR>(buf, f, lane);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      if (f + AH < 16) fr[(f + AH) % (AH + 1)] = lds_frag<TR>(buf, f + AH, lane);
      acc[f & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % (AH + 1)], b, acc[f & 3], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[m][j];
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

// The softmax's VALU work beside the MFMAs.  8 waves; waves w and w + 4 run on the same
// SIMD.  Per pass, an MFMA wave issues 4 bf16 MFMAs (4 chains) and an exponential wave 4
// exp2 with 4 adds into running sums (4 chains), the attention kernel's ratio of one
// exponential and one add per MFMA.  MODE 0: waves 0-3 MFMAs only; 1: waves 4-7
// exponentials only; 2: both at once (one wave of each kind per SIMD); 3: waves 0-3 both
// interleaved (MFMA, exp2, add, ...), waves 4-7 idle.  A wave's role is fixed before its
// loop, so every loop is straight-line code of one kind.
template <bool MF, bool EX>
__device__ __forceinline__ float overlap_loop(const float* seed, int lane, int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)seed[(lane + i) & 63];
    b[i] = (__bf16)seed[(lane + 3 * i) & 63];
  }
  f32x16_t acc[4] = {};
  float x[4], sum[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[k] = seed[(lane + k) & 63] - 1.0f;   // exponents in [-1, 0)
    sum[k] = 0.0f;
  }
  const float step = seed[lane] * 1e-7f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (MF) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
      if (EX) {
        sum[k] += __builtin_amdgcn_exp2f(x[k]);
        x[k] -= step;
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s += sum[k];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  }
  return s;
}

template <int MODE>
__global__ __launch_bounds__(512) void k_overlap(const float* seed, float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float s;
  if (wave < 4) {
    if (MODE == 1) return;
    s = MODE == 3 ? overlap_loop<true, true>(seed, lane, iters) : overlap_loop<true, false>(seed, lane, iters);
  } else {
    if (MODE != 1 && MODE != 2) return;
    s = overlap_loop<false, true>(seed, lane, iters);
  }
  if (s == 1234.5f) sink[blockIdx.x] = s;
}

extern "C" {

// FP8 = 0: bf16 32x32x16; 1: fp8 32x32x64.  blocks x 512 threads (8 waves), iters x 4
// MFMAs per wave.  Returns 0 or a hipError_t.
int mb_mfma_loop(int fp8, int blocks, int iters, const float* seed, float* sink, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(k_mfma_loop<true>, dim3(blocks), dim3(512), 0, s, seed, sink, iters);
  else
    hipLaunchKernelGGL(k_mfma_loop<false>, dim3(blocks), dim3(512), 0, s, seed, sink, iters);
  return (int)hipGetLastError();
}

int mb_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  const int64_t n = bytes / 16, half = (n + 1) / 2;
  hipLaunchKernelGGL(k_copy, dim3((unsigned)((half + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

// five inputs of `bytes` each, laid out one after another at `src`; one output of `bytes`
int mb_copy5(const void* src, void* dst, int64_t bytes, void* stream) {
  const uint4* p = static_cast<const uint4*>(src);
  const int64_t n = bytes / 16;
  hipLaunchKernelGGL(k_copy5, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), p, p + n, p + 2 * n, p + 3 * n, p + 4 * n,
                     static_cast<uint4*>(dst), n);
  return (int)hipGetLastError();
}

// tr = 0: ds_read_b128 fragments, 1: ds_read_b64_tr_b16 pairs.  blocks x 512 threads,
// iters x 16 MFMAs per wave.
int mb_mfma_lds(int tr, int blocks, int iters, const float* seed, float* sink, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (tr)
    hipLaunchKernelGGL(k_mfma_lds<true>, dim3(blocks), dim3(512), 0, s, seed, sink, iters);
  else
    hipLaunchKernelGGL(k_mfma_lds<false>, dim3(blocks), dim3(512), 0, s, seed, sink, iters);
  return (int)hipGetLastError();
}

// mode 0..3 as k_overlap; blocks x 512 threads, iters passes.
int mb_overlap(int mode, int blocks, int iters, const float* seed, float* sink, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(k_overlap<0>, dim3(blocks), dim3(512), 0, s, seed, sink, iters); break;
    case 1: hipLaunchKernelGGL(k_overlap<1>, dim3(blocks), dim3(512), 0, s, seed, sink, iters); break;
    case 2: hipLaunchKernelGGL(k_overlap<2>, dim3(blocks), dim3(512), 0, s, seed, sink, iters); break;
    case 3: hipLaunchKernelGGL(k_overlap<3>, dim3(blocks), dim3(512), 0, s, seed, sink, iters); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// sink: >= 1024 words
int mb_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const int64_t n = bytes / 16, half = (n + 1) / 2;
  hipLaunchKernelGGL(k_read, dim3((unsigned)((half + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), sink, n);
  return (int)hipGetLastError();
}

}  // extern "C"
