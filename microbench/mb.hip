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

// sink: >= 1024 words
int mb_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  const int64_t n = bytes / 16, half = (n + 1) / 2;
  hipLaunchKernelGGL(k_read, dim3((unsigned)((half + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), sink, n);
  return (int)hipGetLastError();
}

}  // extern "C"
