// Shared device helpers for the gfx950 decoder-step kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define QD_WAVE 64

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// f32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two f32 -> their bf16 patterns packed (a in the low half), round to
// nearest even; gfx950 does this in one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)a, (__bf16)b});
}
// hi/lo split of a pair: h = rne(x), l = rne(x - h), packed as above.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& h, uint32_t& l) {
  h = bf16x2_rne(a, b);
  l = bf16x2_rne(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// KV-cache elements: f32 as computed, or bf16 (nearest, ties to even) for the
// half-size cache.  ld_kv4 reads 4 consecutive elements as f32; st_kv stores
// one; kv_round is the value a store then a load gives back.
__device__ __forceinline__ f32x4 ld_kv4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld_kv4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
}
__device__ __forceinline__ void st_kv(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_kv(uint16_t* p, float v) { *p = (uint16_t)bf16_rne(v); }
template <typename KVT>
__device__ __forceinline__ float kv_round(float v) {
  if constexpr (sizeof(KVT) == 2) return __uint_as_float(bf16_rne(v) << 16);
  return v;
}

// Lane exchange within rows of 16 lanes through DPP (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7 - i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15 - i within each 16

// Sum over the 64 lanes of a wave (all lanes active); every lane receives the
// total.  Fixed order: pairs, quads, halves and rows of 16 by DPP, then the
// four rows.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppQuadSwap1>(v);
  v += dpp_f<kDppQuadSwap2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// Sum / maximum over aligned groups of WIDTH lanes (2, 4, 8 or 16), all lanes
// active; every lane of a group receives its group's result.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "group width");
  v += dpp_f<kDppQuadSwap1>(v);
  if (WIDTH >= 4) v += dpp_f<kDppQuadSwap2>(v);
  if (WIDTH >= 8) v += dpp_f<kDppRowHalfMirror>(v);
  if (WIDTH >= 16) v += dpp_f<kDppRowMirror>(v);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
  static_assert(WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16, "group width");
  v = fmaxf(v, dpp_f<kDppQuadSwap1>(v));
  if (WIDTH >= 4) v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
  if (WIDTH >= 8) v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  if (WIDTH >= 16) v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return v;
}

// Maximum over the 64 lanes of a wave (all lanes active), to every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
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

