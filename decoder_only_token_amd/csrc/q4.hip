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

// ---------------------------------------------------------------------------
// Single-row int4 GEMV on the int8 matrix cores (decode).  A block owns R =
// 16 / RG output rows of NS matrices (1, or 2 for gate and up); its W waves
// take the rows' 128-column groups RG at a time (a super-slot; super-slot gs to
// wave gs % W).  The input row h (gain * x / rms(x) for the normed
// projections) is written as y = u (a + b / 128 + c / 16384) with one power of
// two u per block (its largest |y| lies in [32 u, 64 u)) and a, b, c the
// rounded seven-bit digits: |error| <= u / 32768, at most 2^-20 of the row's
// largest input.  In v_mfma_i32_16x16x64_i8, B column n is row n % R of the
// block over group RG gs + n / R (its codes, 16 q, exact), and A row 4 p + j
// is piece p of the input over group RG gs + j (rows with p = 3 or j >= RG,
// and groups past K, read a record of zeros); so D[4 p + n / R][n] is piece
// p's dot product for column n, in lanes 16 p + n.  A super-slot is two such
// products, over the even and the odd columns.  The pieces' sums are weighted
// (1, 2^-7, 2^-14, times u / 16), added across lanes with the row swaps, and
// the W waves' and RG sub-groups' partials of each row added in a fixed order.
// LDS layout per group: [parity e][piece p][quarter q][16 bytes], byte 4 m + t
// of quarter q being column 128 g + 32 q + 8 m + 2 t + e.
constexpr int kGroupBytes = 384;

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Low bytes of four words, packed (w0 in byte 0).
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x0c0c0400u);  // [w0.b0, w1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(w3, w2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

template <int NS, int W, int MS, int MI, int RG>
__global__ __launch_bounds__(64 * W) void k_gemv_q4m(const uint8_t* __restrict__ C0, const uint16_t* __restrict__ S0,
                                                      const uint8_t* __restrict__ C1, const uint16_t* __restrict__ S1,
                                                      int N, int K, const float* __restrict__ x,
                                                      const float* __restrict__ gain, float eps,
                                                      const float* __restrict__ bias, float* __restrict__ y,
                                                      int accumulate) {
  constexpr int NT = 64 * W, R = 16 / RG;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float red[W];
  __shared__ float part[W][NS][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, quarter = lane >> 4;
  const int ng = K / 128, nss = (ng + RG - 1) / RG, r0 = blockIdx.x * R;
  const int row = min(r0 + l16 % R, N - 1), sub = l16 / R;
  // ---- 1. the input (and gains): items of 8 columns, item i = tid + NT j,
  // requested before the codes (reads past K are zeros)
  f32x4 xv[MI][2], gv[MI][2];
  {
    const __amdgpu_buffer_rsrc_t rx = byte_record(x, K * 4);
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int off = (tid + NT * j) * 32;
      xv[j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      xv[j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0));
    }
    if (gain) {
      const __amdgpu_buffer_rsrc_t rg = byte_record(gain, K * 4);
#pragma unroll
      for (int j = 0; j < MI; ++j) {
        const int off = (tid + NT * j) * 32;
        gv[j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
        gv[j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off + 16, 0, 0));
      }
    }
  }
  // ---- 2. the lane's codes and scales: row `row`, quarter `quarter` of
  // group RG gs + sub (past K: the record's zeros)
  u32x4 cw[NS][MS];
  uint16_t sw[NS][MS];
  {
    const __amdgpu_buffer_rsrc_t rc0 = byte_record(C0, N * (K / 2)), rs0 = byte_record(S0, N * ng * 2);
    const __amdgpu_buffer_rsrc_t rc1 = byte_record(NS == 2 ? C1 : C0, N * (K / 2));
    const __amdgpu_buffer_rsrc_t rs1 = byte_record(NS == 2 ? S1 : S0, N * ng * 2);
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int g = (wave + W * j) * RG + sub;
      int oc = g < ng ? row * (K / 2) + g * 64 + quarter * 16 : kPastRecord;
      int os = g < ng ? (row * ng + g) * 2 : kPastRecord;
      asm volatile("" : "+v"(oc), "+v"(os));  // (opaque: one load each, no branch)
      cw[0][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc0, oc, 0, 2 /* streamed */));
      sw[0][j] = __builtin_amdgcn_raw_buffer_load_b16(rs0, os, 0, 0);
      if (NS == 2) {
        cw[NS - 1][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc1, oc, 0, 2));
        sw[NS - 1][j] = __builtin_amdgcn_raw_buffer_load_b16(rs1, os, 0, 0);
      }
    }
  }
  // ---- 3. the row's RMS scale, h, its largest magnitude and u
  float r = 1.f;
  if (gain) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const f32x4 v = xv[j][hh];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    float t = wave_sum(ss);
    if (lane == 0) red[wave] = t;
    __syncthreads();
    t = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) t += red[w];
    r = 1.0f / sqrtf(t / (float)K + eps);
    __syncthreads();
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < MI; ++j)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x4 v = xv[j][hh];
      if (gain) v = v * r * gv[j][hh];
      xv[j][hh] = v;
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) mx = fmaxf(mx, red[w]);
  const int E = (int)((__float_as_uint(mx) >> 23) & 0xFF);  // mx in [2^(E-127), 2^(E-126))
  const bool live = E >= 6;  // inputs below 2^-121 (or all zero) are taken as zero
  const float up = __uint_as_float((uint32_t)(live ? 259 - E : 127) << 23);  // 1 / u = 2^(132 - E)
  const float u16 = live ? ldexpf(1.0f, E - 136) : 0.f;                    // u / 16
  // ---- 4. the pieces into LDS.  v + 1.5 * 2^23 holds rint(v) in its low
  // mantissa bits (|v| <= 64), so its low byte is the digit, two's complement.
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int it = tid + NT * j, col = it * 8;
    if (col < K) {
      const float kMagic = 12582912.0f;
      const float yv[8] = {xv[j][0].x, xv[j][0].y, xv[j][0].z, xv[j][0].w,
                           xv[j][1].x, xv[j][1].y, xv[j][1].z, xv[j][1].w};
      uint32_t dg[3][8];  // [piece][column]: the digit in the low byte
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float v = live ? yv[k] * up : 0.f;  // |v| < 64, exact
        const float ta = v + kMagic, ra = (v - (ta - kMagic)) * 128.0f;
        const float tb = ra + kMagic, rb = (ra - (tb - kMagic)) * 128.0f;
        const float tc = rb + kMagic;
        dg[0][k] = __float_as_uint(ta);
        dg[1][k] = __float_as_uint(tb);
        dg[2][k] = __float_as_uint(tc);
      }
      const int g = col >> 7, qq = (col >> 5) & 3, m = (col >> 3) & 3;
      uint8_t* d = lds + g * kGroupBytes + qq * 16 + m * 4;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        *reinterpret_cast<uint32_t*>(d + p * 64) = pack_low_bytes(dg[p][0], dg[p][2], dg[p][4], dg[p][6]);
        *reinterpret_cast<uint32_t*>(d + 192 + p * 64) = pack_low_bytes(dg[p][1], dg[p][3], dg[p][5], dg[p][7]);
      }
    }
  }
  if (tid < kGroupBytes / 16)  // the record of zeros
    reinterpret_cast<u32x4*>(lds + ng * kGroupBytes)[tid] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  // ---- 5. the super-slots on the matrix cores
  const int ap = l16 >> 2, aj = l16 & 3;  // this lane's A row: piece ap of sub-group aj
  const bool plane = ap < 3 && aj < RG;
  const int abase = ap * 64 + quarter * 16, azero = ng * kGroupBytes;
  float tot[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) tot[s] = 0.f;
#pragma unroll
  for (int j = 0; j < MS; ++j) {
    const int gs = wave + W * j;
    if (gs < nss) {  // wave-uniform
      const int ga = gs * RG + aj;
      const int ao = plane && ga < ng ? ga * kGroupBytes + abase : azero;
      const u32x4 ae = *reinterpret_cast<const u32x4*>(lds + ao);
      const u32x4 aod = *reinterpret_cast<const u32x4*>(lds + ao + 192);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 w = cw[s][j];
        u32x4 be, bo;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          be[k] = ((w[k] << 4) ^ 0x88888880u) & 0xF0F0F0F0u;
          bo[k] = (w[k] ^ 0x88888888u) & 0xF0F0F0F0u;
        }
        i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, ae),
                                                          __builtin_bit_cast(i32x4, be), i32x4{0, 0, 0, 0}, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, aod), __builtin_bit_cast(i32x4, bo),
                                                    acc, 0, 0, 0);
        const int dv = RG == 1 ? acc.x : RG == 2 ? (sub ? acc.y : acc.x)
                                                 : (sub == 0 ? acc.x : sub == 1 ? acc.y : sub == 2 ? acc.z : acc.w);
        tot[s] = fmaf((float)dv, f16_bits_to_f(sw[s][j]), tot[s]);
      }
    }
  }
  // ---- 6. pieces weighted and added across the lane groups; the partials
  const float pw = (lane < 16 ? 1.0f : lane < 32 ? 0.0078125f : lane < 48 ? 6.103515625e-05f : 0.0f) * u16;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float v = tot[s] * pw;
    auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float v2 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
    const float v4 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
    if (lane < 16) part[wave][s][lane] = v4;
  }
  __syncthreads();
  if (tid < R && r0 + tid < N) {
    float t[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      t[s] = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w)
#pragma unroll
        for (int jj = 0; jj < RG; ++jj) t[s] += part[w][s][tid + R * jj];
    }
    const int n = r0 + tid;
    if (NS == 2) {
      y[n] = silu_f(t[0]) * t[NS - 1];
    } else {
      const float v = t[0] + (bias ? bias[n] : 0.f);
      y[n] = accumulate ? y[n] + v : v;
    }
  }
}

template <int NS, int W, int MS, int MI, int RG>
void launch_q4m(hipStream_t s, const uint8_t* c0, const uint16_t* s0, const uint8_t* c1, const uint16_t* s1, int N,
                int K, const float* x, const float* gain, float eps, const float* bias, float* y, int accumulate) {
  const size_t lds = (size_t)(K / 128 + 1) * kGroupBytes;
  hipLaunchKernelGGL((k_gemv_q4m<NS, W, MS, MI, RG>), dim3((N + 16 / RG - 1) / (16 / RG)), dim3(64 * W), lds, s, c0,
                     s0, c1, s1, N, K, x, gain, eps, bias, y, accumulate);
}

// Multi-row form (2 to TM input rows, TM = 8, or 4 for the longest rows;
// speculative verification, short prefills): the rows' digits sit side by
// side in LDS (input row t at
// t * ng * 384 bytes) and every code and scale is requested once and serves
// every row.  A row 4 p + j holds digit p of input row tg * TG + j % TG over
// group RG s + j / TG (TG = 4 / RG rows per product, tg the product's row
// pass), so D[4 p + (n / R) TG + i][n] is digit p's dot product of input
// row tg TG + i with column n.  One power of two u per input row.
template <int NS, int W, int MS, int MI, int RG, int TM>
__global__ __launch_bounds__(64 * W) void k_gemv_q4mr(const uint8_t* __restrict__ C0, const uint16_t* __restrict__ S0,
                                                       const uint8_t* __restrict__ C1, const uint16_t* __restrict__ S1,
                                                       int N, int K, const float* __restrict__ x, int ldx, int T,
                                                       const float* __restrict__ gain, float eps,
                                                       const float* __restrict__ bias, float* __restrict__ y, int ldy,
                                                       int accumulate) {
  constexpr int NT = 64 * W, R = 16 / RG, TG = 4 / RG;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ float red[W][TM];
  __shared__ float part[W][NS][TM][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15, quarter = lane >> 4;
  const int ng = K / 128, nss = (ng + RG - 1) / RG, r0 = blockIdx.x * R;
  const int row = min(r0 + l16 % R, N - 1), sub = l16 / R;
  const int rstride = ng * kGroupBytes;  // LDS bytes of one input row's digits
  // ---- 1. the T input rows (rows past T: an empty record, zeros) and gains
  f32x4 xv[TM][MI][2], gv[MI][2];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const __amdgpu_buffer_rsrc_t rx = byte_record(x + (size_t)min(t, T - 1) * ldx, t < T ? K * 4 : 0);
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int off = (tid + NT * j) * 32;
      xv[t][j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      xv[t][j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16, 0, 0));
    }
  }
  if (gain) {
    const __amdgpu_buffer_rsrc_t rg = byte_record(gain, K * 4);
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int off = (tid + NT * j) * 32;
      gv[j][0] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
      gv[j][1] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, off + 16, 0, 0));
    }
  }
  // ---- 2. the lane's codes and scales, as in the single-row form
  u32x4 cw[NS][MS];
  uint16_t sw[NS][MS];
  {
    const __amdgpu_buffer_rsrc_t rc0 = byte_record(C0, N * (K / 2)), rs0 = byte_record(S0, N * ng * 2);
    const __amdgpu_buffer_rsrc_t rc1 = byte_record(NS == 2 ? C1 : C0, N * (K / 2));
    const __amdgpu_buffer_rsrc_t rs1 = byte_record(NS == 2 ? S1 : S0, N * ng * 2);
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const int g = (wave + W * j) * RG + sub;
      int oc = g < ng ? row * (K / 2) + g * 64 + quarter * 16 : kPastRecord;
      int os = g < ng ? (row * ng + g) * 2 : kPastRecord;
      asm volatile("" : "+v"(oc), "+v"(os));  // (opaque: one load each, no branch)
      cw[0][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc0, oc, 0, 2 /* streamed */));
      sw[0][j] = __builtin_amdgcn_raw_buffer_load_b16(rs0, os, 0, 0);
      if (NS == 2) {
        cw[NS - 1][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc1, oc, 0, 2));
        sw[NS - 1][j] = __builtin_amdgcn_raw_buffer_load_b16(rs1, os, 0, 0);
      }
    }
  }
  // ---- 3. every row's RMS scale, h, largest magnitude and u
  float rr[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) rr[t] = 1.f;
  if (gain) {
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < MI; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x4 v = xv[t][j][hh];
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      ss = wave_sum(ss);
      if (lane == 0) red[wave][t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      float q = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) q += red[w][t];
      rr[t] = 1.0f / sqrtf(q / (float)K + eps);
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        f32x4 v = xv[t][j][hh];
        if (gain) v = v * rr[t] * gv[j][hh];
        xv[t][j][hh] = v;
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
      }
    mx = wave_max(mx);
    if (lane == 0) red[wave][t] = mx;
  }
  __syncthreads();
  float up[TM], u16[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    float mx = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) mx = fmaxf(mx, red[w][t]);
    const int E = (int)((__float_as_uint(mx) >> 23) & 0xFF);
    const bool live = E >= 6 && t < T;
    up[t] = __uint_as_float((uint32_t)(live ? 259 - E : 127) << 23);
    u16[t] = live ? ldexpf(1.0f, E - 136) : 0.f;
    if (!live) up[t] = 0.f;
  }
  // ---- 4. every row's digits into LDS (as in the single-row form)
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t >= T) break;  // uniform
#pragma unroll
    for (int j = 0; j < MI; ++j) {
      const int it = tid + NT * j, col = it * 8;
      if (col < K) {
        const float kMagic = 12582912.0f;
        const float yv[8] = {xv[t][j][0].x, xv[t][j][0].y, xv[t][j][0].z, xv[t][j][0].w,
                             xv[t][j][1].x, xv[t][j][1].y, xv[t][j][1].z, xv[t][j][1].w};
        uint32_t dg[3][8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float v = yv[k] * up[t];  // |v| < 64, exact
          const float ta = v + kMagic, ra = (v - (ta - kMagic)) * 128.0f;
          const float tb = ra + kMagic, rb = (ra - (tb - kMagic)) * 128.0f;
          const float tc = rb + kMagic;
          dg[0][k] = __float_as_uint(ta);
          dg[1][k] = __float_as_uint(tb);
          dg[2][k] = __float_as_uint(tc);
        }
        const int g = col >> 7, qq = (col >> 5) & 3, m = (col >> 3) & 3;
        uint8_t* d = lds + t * rstride + g * kGroupBytes + qq * 16 + m * 4;
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          *reinterpret_cast<uint32_t*>(d + p * 64) = pack_low_bytes(dg[p][0], dg[p][2], dg[p][4], dg[p][6]);
          *reinterpret_cast<uint32_t*>(d + 192 + p * 64) = pack_low_bytes(dg[p][1], dg[p][3], dg[p][5], dg[p][7]);
        }
      }
    }
  }
  if (tid < kGroupBytes / 16)  // the record of zeros, after the T rows
    reinterpret_cast<u32x4*>(lds + T * rstride)[tid] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  // ---- 5. the super-slots on the matrix cores, TG input rows per product
  const int ap = l16 >> 2, aj = l16 & 3;  // A row: digit ap, sub-group aj / TG, row aj % TG of the pass
  const int asub = aj / TG, at = aj % TG;
  const int abase = ap * 64 + quarter * 16, azero = T * rstride;
  float tot[NS][TM];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < TM; ++t) tot[s][t] = 0.f;
#pragma unroll
  for (int j = 0; j < MS; ++j) {
    const int gs = wave + W * j;
    if (gs < nss) {  // wave-uniform
      u32x4 be[NS], bo[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          be[s][k] = ((cw[s][j][k] << 4) ^ 0x88888880u) & 0xF0F0F0F0u;
          bo[s][k] = (cw[s][j][k] ^ 0x88888888u) & 0xF0F0F0F0u;
        }
      const int ga = gs * RG + asub;
#pragma unroll
      for (int tg = 0; tg < TM / TG; ++tg) {
        if (tg * TG >= T) break;  // uniform
        const int ta = tg * TG + at;
        const int ao = ap < 3 && ta < T && ga < ng ? ta * rstride + ga * kGroupBytes + abase : azero;
        const u32x4 ae = *reinterpret_cast<const u32x4*>(lds + ao);
        const u32x4 aod = *reinterpret_cast<const u32x4*>(lds + ao + 192);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, ae),
                                                            __builtin_bit_cast(i32x4, be[s]), i32x4{0, 0, 0, 0}, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, aod), __builtin_bit_cast(i32x4, bo[s]),
                                                      acc, 0, 0, 0);
          const float sc = f16_bits_to_f(sw[s][j]);
#pragma unroll
          for (int i = 0; i < TG; ++i) {
            const int c = sub * TG + i;  // this lane's column's result for row tg TG + i
            const int dv = RG == 1 ? acc[i] : c == 0 ? acc.x : c == 1 ? acc.y : c == 2 ? acc.z : acc.w;
            tot[s][tg * TG + i] = fmaf((float)dv, sc, tot[s][tg * TG + i]);
          }
        }
      }
    }
  }
  // ---- 6. digits weighted and added across the lane groups; the partials
  const float pd = lane < 16 ? 1.0f : lane < 32 ? 0.0078125f : lane < 48 ? 6.103515625e-05f : 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t >= T) break;  // uniform
      const float v = tot[s][t] * pd * u16[t];
      auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      const float v2 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
      const float v4 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      if (lane < 16) part[wave][s][t][lane] = v4;
    }
  __syncthreads();
  if (tid < R * T) {
    const int t = tid / R, rr2 = tid % R, n = r0 + rr2;
    if (n < N) {
      float v[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        v[s] = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w)
#pragma unroll
          for (int jj = 0; jj < RG; ++jj) v[s] += part[w][s][t][rr2 + R * jj];
      }
      float* yo = y + (size_t)t * ldy + n;
      if (NS == 2) {
        *yo = silu_f(v[0]) * v[NS - 1];
      } else {
        const float o = v[0] + (bias ? bias[n] : 0.f);
        *yo = accumulate ? *yo + o : o;
      }
    }
  }
}

template <int NS, int W, int MS, int MI, int RG, int TM>
void launch_q4mr(hipStream_t s, const uint8_t* c0, const uint16_t* s0, const uint8_t* c1, const uint16_t* s1, int N,
                 int K, const float* x, int ldx, int T, const float* gain, float eps, const float* bias, float* y,
                 int ldy, int accumulate) {
  const size_t lds = ((size_t)T * (K / 128) + 1) * kGroupBytes;
  // (more than 64 KiB of LDS for the longest rows: allowed once per kernel;
  // at most 4 rows of 96 groups or 8 rows of 16)
  static const bool big_lds = hipFuncSetAttribute((const void*)k_gemv_q4mr<NS, W, MS, MI, RG, TM>,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (int)(((size_t)4 * 96 + 1) * kGroupBytes)) == hipSuccess;
  (void)big_lds;
  hipLaunchKernelGGL((k_gemv_q4mr<NS, W, MS, MI, RG, TM>), dim3((N + 16 / RG - 1) / (16 / RG)), dim3(64 * W), lds, s, c0,
                     s0, c1, s1, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate);
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

// Single-row GEMVs on the matrix cores: false when the shape is not covered
// (the caller then uses the f32 GEMV).  Rows per block: 8 when that gives
// every CU a block or K is long, else 4 (more blocks for short matrices).
bool q4m_gemv(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x,
              const float* gain, float eps, const float* bias, float* y, int accumulate) {
  const int ng = K / 128;
  if (K % 128 || ng > 96) return false;
  if (ng > 16)
    launch_q4m<1, 8, 6, 3, 2>(s, codes, scales, nullptr, nullptr, N, K, x, gain, eps, bias, y, accumulate);
  else if ((N + 7) / 8 >= 256)
    launch_q4m<1, 8, 1, 1, 2>(s, codes, scales, nullptr, nullptr, N, K, x, gain, eps, bias, y, accumulate);
  else
    launch_q4m<1, 4, 1, 1, 4>(s, codes, scales, nullptr, nullptr, N, K, x, gain, eps, bias, y, accumulate);
  return true;
}

bool q4m_gateup(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su, int N,
                int K, const float* x, const float* gain, float eps, float* a) {
  if (K % 128 || K > 2048) return false;
  launch_q4m<2, 4, 4, 1, 1>(s, cg, sg, cu, su, N, K, x, gain, eps, nullptr, a, 0);
  return true;
}

// Rows per launch of the multi-row forms for K columns: 8 up to 2048 columns,
// 4 up to 12288 (not gate/up: LDS), 0 when not covered.
int q4mr_rows(int K, bool gateup) {
  if (K % 128) return 0;
  return K / 128 <= 16 ? 8 : !gateup && K / 128 <= 96 ? 4 : 0;
}

// Multi-row forms (2 <= T <= q4mr_rows(K) rows): false when the shape is not covered.
bool q4mr_gemv(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
               int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate) {
  const int ng = K / 128;
  if (T < 2 || T > q4mr_rows(K, false)) return false;
  // (the 8-row forms hold more registers: fewer workgroups per CU; up to 4
  // rows the 4-row forms)
#define QD_Q4MR(W_, MS_, MI_, RG_, TM_)                                                                          \
  launch_q4mr<1, W_, MS_, MI_, RG_, TM_>(s, codes, scales, nullptr, nullptr, N, K, x, ldx, T, gain, eps, bias, y, \
                                         ldy, accumulate)
  if (ng > 16) QD_Q4MR(8, 6, 3, 2, 4);
  else if ((N + 7) / 8 >= 256 && T <= 4) QD_Q4MR(8, 1, 1, 2, 4);
  else if ((N + 7) / 8 >= 256) QD_Q4MR(8, 1, 1, 2, 8);
  else if (T <= 4) QD_Q4MR(4, 1, 1, 4, 4);
  else QD_Q4MR(4, 1, 1, 4, 8);
#undef QD_Q4MR
  return true;
}

bool q4mr_gateup(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su, int N,
                 int K, const float* x, int ldx, int T, const float* gain, float eps, float* a, int lda) {
  if (T < 2 || T > q4mr_rows(K, true)) return false;
  if (T <= 4) launch_q4mr<2, 4, 4, 1, 1, 4>(s, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, nullptr, a, lda, 0);
  else launch_q4mr<2, 4, 4, 1, 1, 8>(s, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, nullptr, a, lda, 0);
  return true;
}

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
