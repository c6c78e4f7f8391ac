// Q8_0 projection weights: the quantiser that runs while weights are loaded,
// and the GEMVs of decode and short prefills that widen the codes in
// registers.
//
// "SuperKittens pull request #7", the commit adding the Q8_0 weight dtype
// (ggml type 8) and its matvec: int8 weights in blocks of 32 consecutive
// input columns with one fp16 scale.  For output row n and block b (columns
// 32 b .. 32 b + 31):
//   d    = fp16(absmax / 127)          f32 divide, round to nearest even
//   code = rint(w / d) in [-127, 127]  f32 divide, ties to even; 0 when d = 0
// and the model's weight is code * d.
//
// Layout (private to the library): codes int8 [N][K] row-major; scales fp16
// bit patterns [N][K / 32].  A 16-byte load holds 16 consecutive columns of
// one block.
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kBlock = 32;  // columns per scale
constexpr int kPass = 1024; // columns per pass: 64 lanes x 16 codes

// One wave per two (row, block) items; lane l quantises column 32 (item) + (l % 32).
__global__ __launch_bounds__(256) void k_quantize_q8(const uint16_t* __restrict__ src, int nrows, int K,
                                                     int8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int blocks = K / kBlock;
  const int item = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 2 + ((threadIdx.x >> 5) & 1), l = threadIdx.x & 31;
  const bool live = item < nrows * blocks;  // (every lane still takes part in the reductions)
  const int n = live ? item / blocks : 0, b = live ? item % blocks : 0;
  const float w = live ? bf16_to_f(src[(size_t)n * K + b * kBlock + l]) : 0.f;
  float amax = fabsf(w);
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
  const __half sh = __float2half_rn(amax / 127.0f);
  const float s = __half2float(sh);
  int q = 0;
  if (s > 0.f) q = (int)fminf(fmaxf(rintf(w / s), -127.f), 127.f);
  if (!live) return;
  codes[(size_t)n * K + b * kBlock + l] = (int8_t)q;
  if (l == 0) scales[(size_t)n * blocks + b] = __half_as_ushort(sh);
}

__device__ __forceinline__ float f16_bits_to_f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Staged inputs in LDS are permuted so that the 64 lanes of a wave read them
// without bank conflicts: within each 1024-column pass, lane l owns columns
// 16 l .. 16 l + 15 (its 16 bytes of codes), and its j-th quadruple of inputs
// (columns 16 l + 4 j .. + 3) sits at float offset (64 j + l) 4 of the pass.
// Rows of the staged block are q8_stride(K) floats apart.
__host__ __device__ inline int q8_stride(int K) { return (K + kPass - 1) / kPass * kPass; }

__device__ __forceinline__ int q8_perm(int k) {
  const int p = k >> 10, r = k & 1023, l = r >> 4, j = (r >> 2) & 3;
  return (p << 10) + ((j * 64 + l) << 2) + (k & 3);
}

// h[t][perm(k)] = x[t][k] (* g[k] / rms(x[t])) for T rows; K a multiple of 32.
__device__ __forceinline__ void stage_rows_q8(const float* __restrict__ x, int ldx, int T, int K,
                                              const float* __restrict__ gain, float eps, float* h, float* red) {
  const int ks = q8_stride(K);
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (size_t)t * ldx;
    float ss = 0.f;
    for (int k = threadIdx.x * 4; k < K; k += 1024) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(xr + k);
      *reinterpret_cast<f32x4*>(h + t * ks + q8_perm(k)) = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    if (gain) {  // each thread rescales the pieces it stored
      const float r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)K + eps);
      for (int k = threadIdx.x * 4; k < K; k += 1024) {
        f32x4* hp = reinterpret_cast<f32x4*>(h + t * ks + q8_perm(k));
        *hp = *hp * r * *reinterpret_cast<const f32x4*>(gain + k);
      }
    }
  }
  __syncthreads();
}

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
constexpr int kPastRecord = 0x7FFFFFF0;  // an offset past every record here

// Single input row (decode): its pieces (and the norm gains) are requested
// before the weights, so the wait for them does not also wait for the
// weights (loads complete in order); then h[perm(k)] = x[k] (* g[k] /
// rms(x)) is written once.  Thread t holds columns 4 (t + 256 i) .. + 3 for
// i < NI; reads past K come back as zeros.
template <int NI>
struct RowIn {
  f32x4 x[NI], g[NI];
};

template <int NI>
__device__ __forceinline__ void row_in_load(RowIn<NI>& in, const float* x, const float* gain, int K) {
  const __amdgpu_buffer_rsrc_t rx = byte_record(x, K * 4);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    in.x[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (threadIdx.x + i * 256) * 16, 0, 0));
  if (gain) {
    const __amdgpu_buffer_rsrc_t rg = byte_record(gain, K * 4);
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
    if (k < K) *reinterpret_cast<f32x4*>(h + q8_perm(k)) = gain ? in.x[i] * r * in.g[i] : in.x[i];
  }
  __syncthreads();
}

// 16 codes (16 bytes) of row n from column k, and the fp16 scale bits of
// their block; zeros when k >= K.  No branch, so the waits for earlier loads
// keep their in-order counts.
__device__ __forceinline__ void q8_piece(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int n, int k, int K,
                                         u32x4& c, uint16_t& sc) {
  const bool in = k < K;
  int oc = in ? n * K + k : kPastRecord, os = in ? (n * (K / kBlock) + k / kBlock) * 2 : kPastRecord;
  // (an opaque register value: otherwise the select is turned into two loads
  // under a branch)
  asm volatile("" : "+v"(oc), "+v"(os));
  c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 2 /* streamed */));
  sc = __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0);
}

// The lane's 16 staged inputs of one pass (4 quadruples 256 floats apart) and their sum.
__device__ __forceinline__ void load_x16(const float* hp, f32x4* v, float& sx) {
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = *reinterpret_cast<const f32x4*>(hp + j * 256);
    a += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  }
  sx = a;
}

// sum over one lane's 16 columns of code * x: the bytes xor 0x80 are
// u = code + 128 (unsigned, widened by the byte converts), so the sum is
// sum u x - 128 sum x.  Dword m holds columns 4 m .. 4 m + 3.
__device__ __forceinline__ float dot16_q8(u32x4 c, const f32x4* v, float sx) {
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t w = c[m] ^ 0x80808080u;
    const f32x4 a = v[m];
    s = fmaf((float)(w & 0xFF), a.x, s);
    s = fmaf((float)((w >> 8) & 0xFF), a.y, s);
    s = fmaf((float)((w >> 16) & 0xFF), a.z, s);
    s = fmaf((float)(w >> 24), a.w, s);
  }
  return fmaf(-128.0f, sx, s);
}

// y[t][n] (=|+=) sum_b d[n][b] sum_{k in b} code[n][k] h[t][k] (+ bias[n])
// for T <= TM rows.  Each wave owns RPW output rows; in each 1024-column pass
// a lane takes 16 bytes (16 codes, half a block) of each row.  The codes of
// NP passes are requested together, so a row of up to NP * 1024 columns costs
// one HBM round trip; with TM = 1 the input row is requested before them
// (rows of up to 16384 columns).
template <int RPW, int TM, int NP>
__global__ __launch_bounds__(256) void k_gemv_q8(const int8_t* __restrict__ C8, const uint16_t* __restrict__ S8,
                                                 int N, int K, const float* __restrict__ x, int ldx, int T,
                                                 const float* __restrict__ gain, float eps,
                                                 const float* __restrict__ bias, float* __restrict__ y, int ldy,
                                                 int accumulate) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int ks = q8_stride(K), np = (K + kPass - 1) / kPass;
  u32x4 c[NP][RPW];
  uint16_t sc[NP][RPW];  // fp16 bits, widened where used
  const __amdgpu_buffer_rsrc_t rc = byte_record(C8, N * K), rs = byte_record(S8, N * (K / kBlock) * 2);
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < RPW; ++i) q8_piece(rc, rs, min(n0 + i, N - 1), (pb + p) * kPass + lane * 16, K, c[p][i], sc[p][i]);
  };
  constexpr int NI = NP == 8 ? 16 : NP;  // input pieces per thread: 1024 NI columns
  if (TM == 1 && K <= 1024 * NI) {
    RowIn<NI> in;
    row_in_load(in, x, gain, K);
    load(0);  // (rows past N repeat row N - 1; their waves return after the staging)
    row_in_stage(in, gain != nullptr, K, eps, h, red);
  } else {
    load(0);
    stage_rows_q8(x, ldx, T, K, gain, eps, h, red);
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
      if ((pb + p) * kPass + lane * 16 < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
            f32x4 v[4];
            float sx;
            load_x16(h + t * ks + (pb + p) * kPass + lane * 4, v, sx);
#pragma unroll
            for (int i = 0; i < RPW; ++i) acc[i][t] = fmaf(f16_bits_to_f(sc[p][i]), dot16_q8(c[p][i], v, sx), acc[i][t]);
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

// a[t][n] = SiLU(gate row n . h[t]) * (up row n . h[t]), both rows Q8_0;
// loads as in k_gemv_q8.
template <int RPW, int TM, int NP>
__global__ __launch_bounds__(256) void k_gemv_gateup_q8(const int8_t* __restrict__ Cg, const uint16_t* __restrict__ Sg,
                                                        const int8_t* __restrict__ Cu, const uint16_t* __restrict__ Su,
                                                        int N, int K, const float* __restrict__ x, int ldx, int T,
                                                        const float* __restrict__ gain, float eps,
                                                        float* __restrict__ a, int lda) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int ks = q8_stride(K), np = (K + kPass - 1) / kPass;
  u32x4 cg[NP][RPW], cu[NP][RPW];
  uint16_t sg[NP][RPW], su[NP][RPW];  // fp16 bits, widened where used
  const __amdgpu_buffer_rsrc_t rcg = byte_record(Cg, N * K), rsg = byte_record(Sg, N * (K / kBlock) * 2);
  const __amdgpu_buffer_rsrc_t rcu = byte_record(Cu, N * K), rsu = byte_record(Su, N * (K / kBlock) * 2);
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int n = min(n0 + i, N - 1), k = (pb + p) * kPass + lane * 16;
        q8_piece(rcg, rsg, n, k, K, cg[p][i], sg[p][i]);
        q8_piece(rcu, rsu, n, k, K, cu[p][i], su[p][i]);
      }
  };
  constexpr int NI = NP == 8 ? 16 : NP;  // input pieces per thread: 1024 NI columns
  if (TM == 1 && K <= 1024 * NI) {
    RowIn<NI> in;
    row_in_load(in, x, gain, K);
    load(0);  // (rows past N repeat row N - 1; their waves return after the staging)
    row_in_stage(in, gain != nullptr, K, eps, h, red);
  } else {
    load(0);
    stage_rows_q8(x, ldx, T, K, gain, eps, h, red);
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
      if ((pb + p) * kPass + lane * 16 < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
            f32x4 v[4];
            float sx;
            load_x16(h + t * ks + (pb + p) * kPass + lane * 4, v, sx);
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              ag[i][t] = fmaf(f16_bits_to_f(sg[p][i]), dot16_q8(cg[p][i], v, sx), ag[i][t]);
              au[i][t] = fmaf(f16_bits_to_f(su[p][i]), dot16_q8(cu[p][i], v, sx), au[i][t]);
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
int q8_rpw(int N, int ncu, int max_rpw) {
  int r = max_rpw;
  while (r > 1 && (N + 4 * r - 1) / (4 * r) < 2 * ncu) r >>= 1;
  return r;
}

// Passes requested together: the row's pass count rounded up to 1, 2, 4 or 8.
int q8_np(int K) {
  const int np = (K + kPass - 1) / kPass;
  return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
}

template <int RPW, int NP>
void gemv_q8_np(hipStream_t s, dim3 grid, size_t lds, const int8_t* codes, const uint16_t* scales, int N, int K,
                const float* x, int ldx, int T, const float* gain, float eps, const float* bias, float* y, int ldy,
                int accumulate) {
  if (T == 1)
    hipLaunchKernelGGL((k_gemv_q8<RPW, 1, NP>), grid, dim3(256), lds, s, codes, scales, N, K, x, ldx, T, gain, eps,
                       bias, y, ldy, accumulate);
  else
    hipLaunchKernelGGL((k_gemv_q8<RPW, GEMV_MAX_T, 1>), grid, dim3(256), lds, s, codes, scales, N, K, x, ldx, T, gain,
                       eps, bias, y, ldy, accumulate);
}

template <int RPW>
void gemv_q8_t(hipStream_t s, dim3 grid, size_t lds, const int8_t* codes, const uint16_t* scales, int N, int K,
               const float* x, int ldx, int T, const float* gain, float eps, const float* bias, float* y, int ldy,
               int accumulate) {
  switch (q8_np(K)) {
    case 1: gemv_q8_np<RPW, 1>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    case 2: gemv_q8_np<RPW, 2>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    case 4: gemv_q8_np<RPW, 4>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    default: gemv_q8_np<RPW, 8>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
  }
}

template <int RPW, int NP>
void gateup_q8_np(hipStream_t s, dim3 grid, size_t lds, const int8_t* cg, const uint16_t* sg, const int8_t* cu,
                  const uint16_t* su, int N, int K, const float* x, int ldx, int T, const float* gain, float eps,
                  float* a, int lda) {
  if (T == 1)
    hipLaunchKernelGGL((k_gemv_gateup_q8<RPW, 1, NP>), grid, dim3(256), lds, s, cg, sg, cu, su, N, K, x, ldx, T, gain,
                       eps, a, lda);
  else
    hipLaunchKernelGGL((k_gemv_gateup_q8<RPW, GEMV_MAX_T, 1>), grid, dim3(256), lds, s, cg, sg, cu, su, N, K, x, ldx,
                       T, gain, eps, a, lda);
}

template <int RPW>
void gateup_q8_t(hipStream_t s, dim3 grid, size_t lds, const int8_t* cg, const uint16_t* sg, const int8_t* cu,
                 const uint16_t* su, int N, int K, const float* x, int ldx, int T, const float* gain, float eps,
                 float* a, int lda) {
  switch (q8_np(K)) {
    case 1: gateup_q8_np<RPW, 1>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
    case 2: gateup_q8_np<RPW, 2>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
    case 4: gateup_q8_np<RPW, 4>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
    default: gateup_q8_np<RPW, 8>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda); break;
  }
}

}  // namespace

int q8_gemv_t_tile(int K) {
  int t = (16384 - 64) / q8_stride(K);  // staged rows (plus the reduction slots) within 64 KiB of LDS
  if (t > GEMV_MAX_T) t = GEMV_MAX_T;
  if (t < 1) t = 1;
  return t;
}

void launch_quantize_q8(hipStream_t s, const uint16_t* src, int nrows, int K, int8_t* codes, uint16_t* scales) {
  const int items = nrows * (K / kBlock);
  hipLaunchKernelGGL(k_quantize_q8, dim3((items + 7) / 8), dim3(256), 0, s, src, nrows, K, codes, scales);
}

void launch_gemv_q8(hipStream_t s, const int8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
                    int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate,
                    int ncu) {
  const size_t lds = (8 + (size_t)T * q8_stride(K)) * sizeof(float);
  const int r = q8_rpw(N, ncu, 4);
  const dim3 grid((N + 4 * r - 1) / (4 * r));
  if (r == 4)
    gemv_q8_t<4>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate);
  else if (r == 2)
    gemv_q8_t<2>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate);
  else
    gemv_q8_t<1>(s, grid, lds, codes, scales, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate);
}

void launch_gemv_gateup_q8(hipStream_t s, const int8_t* cg, const uint16_t* sg, const int8_t* cu, const uint16_t* su,
                           int N, int K, const float* x, int ldx, int T, const float* gain, float eps, float* a,
                           int lda, int ncu) {
  const size_t lds = (8 + (size_t)T * q8_stride(K)) * sizeof(float);
  const int r = q8_rpw(N, ncu, 4);
  const dim3 grid((N + 4 * r - 1) / (4 * r));
  if (r == 4)
    gateup_q8_t<4>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
  else if (r == 2)
    gateup_q8_t<2>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
  else
    gateup_q8_t<1>(s, grid, lds, cg, sg, cu, su, N, K, x, ldx, T, gain, eps, a, lda);
}
