// Shared device helpers for the gfx950 decoder-step kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define QD_WAVE 64

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Sum over the 64 lanes of a wave; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, QD_WAVE);
  return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = WIDTH / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, QD_WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, QD_WAVE));
  return v;
}

// Block-wide sum for blockDim.x == 256 (4 waves); all threads get the result.
__device__ __forceinline__ float block_sum_256(float v, float* red /* >= 4 floats of LDS */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Dot of one bf16 weight row chunk (8 values in a u32x4) with 8 staged inputs.
__device__ __forceinline__ float dot8(u32x4 w, const float* hk) {
  f32x4 a = *reinterpret_cast<const f32x4*>(hk);
  f32x4 b = *reinterpret_cast<const f32x4*>(hk + 4);
  float s = bf16_lo(w.x) * a.x;
  s = fmaf(bf16_hi(w.x), a.y, s);
  s = fmaf(bf16_lo(w.y), a.z, s);
  s = fmaf(bf16_hi(w.y), a.w, s);
  s = fmaf(bf16_lo(w.z), b.x, s);
  s = fmaf(bf16_hi(w.z), b.y, s);
  s = fmaf(bf16_lo(w.w), b.z, s);
  s = fmaf(bf16_hi(w.w), b.w, s);
  return s;
}

