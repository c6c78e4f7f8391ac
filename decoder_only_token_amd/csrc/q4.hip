// int4 group-128 projection weights: the quantiser that runs while weights
// are loaded, the decode / short-prefill GEMVs that dequantise in registers,
// and the code layout both share.
//
// "EMBERGLASS (qwen-webgpu-lora) README", "Why it's hard" and "Note on
// weights": projection weights are quantised to symmetric int4 in groups of
// 128 on their way to the GPU.  For output row n and group g (input columns
// 128 g .. 128 g + 127):
//   s    = fp16(absmax / 7)            f32 divide, round to nearest even
//   code = rint(w / s) in [-7, 7]      f32 divide, ties to even; 0 when s = 0
// and the model's weight is code * s.
//
// Layout (private to the library): codes u8 [N][K / 2], byte j of a row holds
// column 2 j in its low nibble and column 2 j + 1 in its high nibble, each as
// code + 8; scales are fp16 bit patterns [N][K / 128].  A 16-byte load holds
// 32 consecutive columns of one group.
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace {

// One wave per (row, group); lane l quantises columns 128 g + 2 l and 2 l + 1.
__global__ __launch_bounds__(256) void k_quantize_q4(const uint16_t* __restrict__ src, int nrows, int K,
                                                     uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int groups = K / 128;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= nrows * groups) return;
  const int n = item / groups, g = item % groups;
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(src + (size_t)n * K + g * 128 + 2 * lane);
  const float w0 = bf16_lo(pair), w1 = bf16_hi(pair);
  const float amax = wave_max(fmaxf(fabsf(w0), fabsf(w1)));
  const __half sh = __float2half_rn(amax / 7.0f);
  const float s = __half2float(sh);
  auto code = [&](float w) -> int {
    if (!(s > 0.f)) return 0;
    const float q = rintf(w / s);
    return (int)fminf(fmaxf(q, -7.f), 7.f);
  };
  const int q0 = code(w0), q1 = code(w1);
  codes[(size_t)n * (K / 2) + g * 64 + lane] = (uint8_t)((q0 + 8) | ((q1 + 8) << 4));
  if (lane == 0) scales[(size_t)n * groups + g] = __half_as_ushort(sh);
}

__device__ __forceinline__ float f16_bits_to_f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Staged inputs in LDS are permuted so that the 64 lanes of a wave read them
// without bank conflicts: within each 2048-column pass, lane l owns columns
// 32 l .. 32 l + 31 (its 16 bytes of codes), and its j-th quadruple of inputs
// (columns 32 l + 4 j .. + 3) sits at float offset (64 j + l) 4 of the pass.
// Extra bf16 rows of a GEMV launch (see gemv_extra_bf16).
struct XRows {
  const uint16_t* W;  // [N][K] bf16, or null
  int N;
  float* y;
  int ldy;
  int blk0;  // first block of the extra rows
};

// Rows of the staged block are q4_stride(K) floats apart.
__host__ __device__ inline int q4_stride(int K) { return (K + 2047) / 2048 * 2048; }

__device__ __forceinline__ int q4_perm(int k) {
  const int p = k >> 11, r = k & 2047, l = r >> 5, j = (r >> 2) & 7;
  return (p << 11) + ((j * 64 + l) << 2) + (k & 3);
}

// h[t][perm(k)] = x[t][k] (* g[k] / rms(x[t])); K a multiple of 128.  Each
// thread requests up to 12 pieces of 16 bytes before storing any.
__device__ __forceinline__ void stage_input_q4(const float* __restrict__ x, int ldx, int T, int K,
                                               const float* __restrict__ gain, float eps, float* h, float* red) {
  constexpr int B = 12;
  const int ks = q4_stride(K);
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (size_t)t * ldx;
    float ss = 0.f;
    for (int k0 = 0; k0 < K; k0 += B * 1024) {
      f32x4 v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int k = k0 + (threadIdx.x + i * 256) * 4;
        if (k < K) v[i] = *reinterpret_cast<const f32x4*>(xr + k);
      }
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int k = k0 + (threadIdx.x + i * 256) * 4;
        if (k < K) {
          *reinterpret_cast<f32x4*>(h + t * ks + q4_perm(k)) = v[i];
          ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        }
      }
    }
    if (gain) {  // each thread rescales the pieces it stored
      const float r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)K + eps);
      for (int k = threadIdx.x * 4; k < K; k += 1024) {
        f32x4* hp = reinterpret_cast<f32x4*>(h + t * ks + q4_perm(k));
        *hp = *hp * r * *reinterpret_cast<const f32x4*>(gain + k);
      }
    }
  }
  __syncthreads();
}

// Single input row (decode): its pieces (and the norm gains) are requested
// into registers before the weights, so the wait for them does not also wait
// for the weights (loads complete in order); then h[perm(k)] = x[k]
// (* g[k] / rms(x)) is written once.  Thread t holds columns 4 (t + 256 i) ..
// + 3 for i < NI; reads past K come back as zeros (buffer record of K floats).
template <int NI>
struct RowIn {
  f32x4 x[NI], g[NI];
};

// A buffer record over `bytes` bytes at `p` (the same in every lane; taken
// from lane 0 so it lives in scalar registers).  Loads at offsets past it
// read zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_record(const void* p, int bytes) {
  const uint64_t v = (uint64_t)p;
  const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_record(const float* p, int n) { return byte_record(p, n * 4); }
constexpr int kPastRecord = 0x7FFFFFF0;  // an offset past every record here

// 16 bytes of codes (32 columns) of row n from column k, and the fp16 scale
// bits of its group; zeros when k >= K.  No branch, so the waits for earlier
// loads keep their in-order counts.
__device__ __forceinline__ void q4_piece(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int n, int k, int K,
                                         u32x4& c, uint16_t& sc) {
  const bool in = k < K;
  int oc = in ? n * (K / 2) + k / 2 : kPastRecord, os = in ? (n * (K / 128) + k / 128) * 2 : kPastRecord;
  // (an opaque register value: otherwise the select is turned into two loads
  // under a branch)
  asm volatile("" : "+v"(oc), "+v"(os));
  c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 2 /* streamed */));
  sc = __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0);
}

template <int NI>
__device__ __forceinline__ void row_in_load(RowIn<NI>& in, const float* x, const float* gain, int K) {
  const __amdgpu_buffer_rsrc_t rx = f32_record(x, K);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    in.x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (threadIdx.x + i * 256) * 16, 0, 0));
  if (gain) {
    const __amdgpu_buffer_rsrc_t rg = f32_record(gain, K);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      in.g[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (threadIdx.x + i * 256) * 16, 0, 0));
  }
}

template <int NI>
__device__ __forceinline__ void row_in_stage(const RowIn<NI>& in, bool gain, int K, float eps, float* h, float* red) {
  float r = 1.f;
  if (gain) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const f32x4 v = in.x[i];
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)K + eps);
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int k = (threadIdx.x + i * 256) * 4;
    if (k < K) *reinterpret_cast<f32x4*>(h + q4_perm(k)) = gain ? in.x[i] * r * in.g[i] : in.x[i];
  }
  __syncthreads();
}

// sum over one lane's 32 columns of code * x, with u = code + 8 in the nibbles:
// sum u x - 8 sum x.  Dword m holds columns 8 m .. 8 m + 7; v[2 m], v[2 m + 1]
// are their inputs.
__device__ __forceinline__ float dot32_q4(u32x4 c, const f32x4* v, float sx) {
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w = c[m];
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f32x4 a = v[2 * m], b = v[2 * m + 1];
    s = fmaf((float)(lo & 0xFF), a.x, s);
    s = fmaf((float)(hi & 0xFF), a.y, s);
    s = fmaf((float)((lo >> 8) & 0xFF), a.z, s);
    s = fmaf((float)((hi >> 8) & 0xFF), a.w, s);
    s = fmaf((float)((lo >> 16) & 0xFF), b.x, s);
    s = fmaf((float)((hi >> 16) & 0xFF), b.y, s);
    s = fmaf((float)(lo >> 24), b.z, s);
    s = fmaf((float)(hi >> 24), b.w, s);
  }
  return fmaf(-8.0f, sx, s);
}

__device__ __forceinline__ void load_x32(const float* hp, f32x4* v, float& sx) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = *reinterpret_cast<const f32x4*>(hp + j * 256);
    a += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  }
  sx = a;
}

// y[t][n] (=|+=) sum_g s[n][g] sum_{k in g} code[n][k] h[t][k] (+ bias[n]) for
// T <= TM rows.  Each wave owns RPW output rows; in each 2048-column pass a
// lane takes 16 bytes (32 codes) of each row.  The codes of NP passes are
// requested together (the first NP before the input is staged), so a row of
// up to NP * 2048 columns costs one HBM round trip.  TM = 1 (decode) keeps
// the register count low enough for several waves per SIMD.
// Blocks blk0 .. of the launch: bf16 rows W [N][K] against the same staged
// input (one row per wave), yx[t][n] = row n . h[t] — the adapter's down
// products beside the q|k|v rows, so they cost no launch of their own.
template <int TM, int NP>
__device__ __forceinline__ void gemv_extra_bf16(const XRows& xr, int K, const float* __restrict__ x, int ldx, int T,
                                                const float* __restrict__ gain, float eps, float* h, float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = ((int)blockIdx.x - xr.blk0) * 4 + wave, ks = q4_stride(K), np = (K + 2047) / 2048;
  const bool live = n < xr.N;
  u32x4 w[NP][4];
  auto load = [&](int pb) {  // 32 columns (64 bytes) of the row per lane and pass
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = (pb + p) * 2048 + lane * 32;
      if (live && pb + p < np && k < K) {
#pragma unroll
        for (int m = 0; m < 4; ++m) w[p][m] = *reinterpret_cast<const u32x4*>(xr.W + (size_t)n * K + k + 8 * m);
      }
    }
  };
  if (TM == 1 && K <= 2048 * NP) {  // (the input pieces cover 2048 NP columns)
    RowIn<2 * NP> in;
    row_in_load(in, x, gain, K);
    load(0);
    row_in_stage(in, gain != nullptr, K, eps, h, red);
  } else {
    load(0);
    stage_input_q4(x, ldx, T, K, gain, eps, h, red);
  }
  if (!live) return;
  float acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) acc[t] = 0.f;
  for (int pb = 0; pb < np; pb += NP) {
    if (pb) load(pb);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (pb + p >= np || (pb + p) * 2048 + lane * 32 >= K) continue;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        if (t >= T) continue;
        f32x4 v[8];
        float sx;
        load_x32(h + t * ks + (pb + p) * 2048 + lane * 4, v, sx);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // dword i of piece m: columns 8 m + 2 i, + 1
            const uint32_t b = w[p][m][i];
            const f32x4 a = v[2 * m + i / 2];
            const float x0 = (i & 1) ? a.z : a.x, x1 = (i & 1) ? a.w : a.y;
            acc[t] = fmaf(__uint_as_float(b << 16), x0, acc[t]);
            acc[t] = fmaf(__uint_as_float(b & 0xFFFF0000u), x1, acc[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < T) {
      const float s = wave_sum(acc[t]);
      if (lane == 0) xr.y[(size_t)t * xr.ldy + n] = s;
    }
  }
}

// XR: the launch has extra bf16 rows (a separate instantiation, so launches
// without them do not carry that path's registers)
template <int RPW, int TM, int NP, bool XR>
__global__ __launch_bounds__(256) void k_gemv_q4(const uint8_t* __restrict__ C4, const uint16_t* __restrict__ S4,
                                                 int N, int K, const float* __restrict__ x, int ldx, int T,
                                                 const float* __restrict__ gain, float eps,
                                                 const float* __restrict__ bias, float* __restrict__ y, int ldy,
                                                 int accumulate, XRows xr) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  if (XR && (int)blockIdx.x >= xr.blk0) {  // block-uniform
    gemv_extra_bf16<TM, NP>(xr, K, x, ldx, T, gain, eps, h, red);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int groups = K / 128, ks = q4_stride(K), np = (K + 2047) / 2048;
  u32x4 c[NP][RPW];
  uint16_t sc[NP][RPW];  // fp16 bits, widened where used (a conversion here would wait for the load)
  const __amdgpu_buffer_rsrc_t rc = byte_record(C4, N * (K / 2)), rs = byte_record(S4, N * groups * 2);
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < RPW; ++i) q4_piece(rc, rs, min(n0 + i, N - 1), (pb + p) * 2048 + lane * 32, K, c[p][i], sc[p][i]);
  };
  if (TM == 1 && K <= 2048 * NP) {  // (the input pieces cover 2048 NP columns)
    RowIn<2 * NP> in;
    row_in_load(in, x, gain, K);
    load(0);  // (rows past N repeat row N - 1; their waves return after the staging)
    row_in_stage(in, gain != nullptr, K, eps, h, red);
  } else {
    if (n0 < N) load(0);
    stage_input_q4(x, ldx, T, K, gain, eps, h, red);
  }
  if (n0 >= N) return;
  float acc[RPW][TM];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[i][t] = 0.f;
  for (int pb = 0; pb < np; pb += NP) {
    if (pb) load(pb);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if ((pb + p) * 2048 + lane * 32 < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
            f32x4 v[8];
            float sx;
            load_x32(h + t * ks + (pb + p) * 2048 + lane * 4, v, sx);
#pragma unroll
            for (int i = 0; i < RPW; ++i) acc[i][t] = fmaf(f16_bits_to_f(sc[p][i]), dot32_q4(c[p][i], v, sx), acc[i][t]);
          }
        }
      }
      // one pass's inputs in registers at a time (hoisting every pass's LDS
      // reads would cost the occupancy)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < T) {
        const float s = wave_sum(acc[i][t]);
        const int n = n0 + i;
        if (lane == 0 && n < N) {
          float* yp = y + (size_t)t * ldy + n;
          const float v = s + (bias ? bias[n] : 0.f);
          *yp = accumulate ? (*yp + v) : v;
        }
      }
    }
  }
}

// a[t][n] = SiLU(gate row n . h[t]) * (up row n . h[t]), both rows int4;
// loads as in k_gemv_q4.
template <int RPW, int TM, int NP>
__global__ __launch_bounds__(256) void k_gemv_gateup_q4(const uint8_t* __restrict__ Cg, const uint16_t* __restrict__ Sg,
                                                        const uint8_t* __restrict__ Cu, const uint16_t* __restrict__ Su,
                                                        int N, int K, const float* __restrict__ x, int ldx, int T,
                                                        const float* __restrict__ gain, float eps,
                                                        float* __restrict__ a, int lda) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int groups = K / 128, ks = q4_stride(K), np = (K + 2047) / 2048;
  u32x4 cg[NP][RPW], cu[NP][RPW];
  uint16_t sg[NP][RPW], su[NP][RPW];  // fp16 bits, widened where used
  const __amdgpu_buffer_rsrc_t rcg = byte_record(Cg, N * (K / 2)), rsg = byte_record(Sg, N * groups * 2);
  const __amdgpu_buffer_rsrc_t rcu = byte_record(Cu, N * (K / 2)), rsu = byte_record(Su, N * groups * 2);
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int n = min(n0 + i, N - 1), k = (pb + p) * 2048 + lane * 32;
        q4_piece(rcg, rsg, n, k, K, cg[p][i], sg[p][i]);
        q4_piece(rcu, rsu, n, k, K, cu[p][i], su[p][i]);
      }
  };
  if (TM == 1 && K <= 2048 * NP) {  // (the input pieces cover 2048 NP columns)
    RowIn<2 * NP> in;
    row_in_load(in, x, gain, K);
    load(0);  // (rows past N repeat row N - 1; their waves return after the staging)
    row_in_stage(in, gain != nullptr, K, eps, h, red);
  } else {
    if (n0 < N) load(0);
    stage_input_q4(x, ldx, T, K, gain, eps, h, red);
  }
  if (n0 >= N) return;
  float ag[RPW][TM], au[RPW][TM];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int t = 0; t < TM; ++t) ag[i][t] = au[i][t] = 0.f;
  for (int pb = 0; pb < np; pb += NP) {
    if (pb) load(pb);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if ((pb + p) * 2048 + lane * 32 < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
            f32x4 v[8];
            float sx;
            load_x32(h + t * ks + (pb + p) * 2048 + lane * 4, v, sx);
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              ag[i][t] = fmaf(f16_bits_to_f(sg[p][i]), dot32_q4(cg[p][i], v, sx), ag[i][t]);
              au[i][t] = fmaf(f16_bits_to_f(su[p][i]), dot32_q4(cu[p][i], v, sx), au[i][t]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < T) {
        const float g = wave_sum(ag[i][t]);
        const float u = wave_sum(au[i][t]);
        const int n = n0 + i;
        if (lane == 0 && n < N) a[(size_t)t * lda + n] = silu_f(g) * u;
      }
    }
  }
}

// Output rows per wave: as many as max_rpw while the grid (four waves per
// block) still gives every CU at least two blocks.
int q4_rpw(int N, int ncu, int max_rpw) {
  int r = max_rpw;
  while (r > 1 && (N + 4 * r - 1) / (4 * r) < 2 * ncu) r >>= 1;
  return r;
}

// Passes requested together: the row's pass count rounded up to 1, 2, 4 or 8.
int q4_np(int K) {
  const int np = (K + 2047) / 2048;
  return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
}

template <int RPW, int NP>
void gemv_q4_np(hipStream_t s, dim3 grid, size_t lds, const uint8_t* codes, const uint16_t* scales, int N, int K,
                const float* x, int ldx, int T, const float* gain, float eps, const float* bias, float* y, int ldy,
                int accumulate, const XRows& xr0) {
  XRows xr = xr0;
  xr.blk0 = (int)grid.x;
  const dim3 g2(grid.x + (xr.W ? (xr.N + 3) / 4 : 0));
#define QD_GEMV_Q4(TM_, NP_, XR_)                                                                                   \
  hipLaunchKernelGGL((k_gemv_q4<RPW, TM_, NP_, XR_>), g2, dim3(256), lds, s, codes, scales, N, K, x, ldx, T, gain, \
                     eps, bias, y, ldy, accumulate, xr)
  if (T == 1) {
    if (xr.W) QD_GEMV_Q4(1, NP, true);
    else QD_GEMV_Q4(1, NP, false);
  } else {
    if (xr.W) QD_GEMV_Q4(GEMV_MAX_T, 1, true);
    else QD_GEMV_Q4(GEMV_MAX_T, 1, false);
  }
#undef QD_GEMV_Q4
}

template <int RPW>
void gemv_q4_t(hipStream_t s, dim3 grid, size_t lds, const uint8_t* codes, const uint16_t* scales, int N, int K,
               const float* x, int ldx, int T, const float* gain, float eps, const float* bias, float* y, int ldy,
               int accumulate, const XRows& xr) {
  switch (q4_np(K)) {
    case 1: gemv_q4_np<RPW, 1>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr); break;
    case 2: gemv_q4_np<RPW, 2>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr); break;
    case 4: gemv_q4_np<RPW, 4>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr); break;
    default: gemv_q4_np<RPW, 8>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr); break;
  }
}

template <int RPW, int NP>
void gateup_q4_np(hipStream_t s, dim3 grid, size_t lds, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu,
                  const uint16_t* su, int N, int K, const float* x, int ldx, int T, const float* gain, float eps,
                  float* a, int lda) {
  if (T == 1)
    hipLaunchKernelGGL((k_gemv_gateup_q4<RPW, 1, NP>), grid, dim3(256), lds, s, cg, sg, cu, su, N, K, x, ldx, T, gain,
                       eps, a, lda);
  else
    hipLaunchKernelGGL((k_gemv_gateup_q4<RPW, GEMV_MAX_T, 1>), grid, dim3(256), lds, s, cg, sg, cu, su, N, K, x, ldx,
                       T, gain, eps, a, lda);
}

template <int RPW>
void gateup_q4_t(hipStream_t s, dim3 grid, size_t lds, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu,
                 const uint16_t* su, int N, int K, const float* x, int ldx, int T, const float* gain, float eps,
                 float* a, int lda) {
  switch (q4_np(K)) {
    case 1: gateup_q4_np<RPW, 1>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
    case 2: gateup_q4_np<RPW, 2>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
    default: gateup_q4_np<RPW, 4>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
  }
}

}  // namespace

int q4_gemv_t_tile(int K) {
  int t = (16384 - 64) / q4_stride(K);  // staged rows (plus the reduction slots) within 64 KiB of LDS
  if (t > GEMV_MAX_T) t = GEMV_MAX_T;
  if (t < 1) t = 1;
  return t;
}

void launch_quantize_q4(hipStream_t s, const uint16_t* src, int nrows, int K, uint8_t* codes, uint16_t* scales) {
  const int items = nrows * (K / 128);
  hipLaunchKernelGGL(k_quantize_q4, dim3((items + 3) / 4), dim3(256), 0, s, src, nrows, K, codes, scales);
}

void launch_gemv_q4(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
                    int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate,
                    int ncu, const uint16_t* xw, int xn, float* xy, int ldxy) {
  const size_t lds = (8 + (size_t)T * q4_stride(K)) * sizeof(float);
  const int r = q4_rpw(N, ncu, 4);
  const dim3 grid((N + 4 * r - 1) / (4 * r));
  const XRows xr{xw, xn, xy, ldxy, 0};
  if (r == 4)
    gemv_q4_t<4>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr);
  else if (r == 2)
    gemv_q4_t<2>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr);
  else
    gemv_q4_t<1>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate, xr);
}

void launch_gemv_gateup_q4(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su,
                           int N, int K, const float* x, int ldx, int T, const float* gain, float eps, float* a,
                           int lda, int ncu) {
  const size_t lds = (8 + (size_t)T * q4_stride(K)) * sizeof(float);
  const int r = q4_rpw(N, ncu, 4);
  const dim3 grid((N + 4 * r - 1) / (4 * r));
  if (r == 4)
    gateup_q4_t<4>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
  else if (r == 2)
    gateup_q4_t<2>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
  else
    gateup_q4_t<1>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
}
