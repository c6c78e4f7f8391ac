// Decoder-step kernels for gfx950 (wave64, 160 KB LDS per CU).
//
// Activations, accumulators and the KV cache are f32; weights are bf16 (or int4
// group-128 codes with fp16 scales) widened in registers.  Every reduction has
// a fixed order (no float atomics), so results are bit-identical run to run.
#include "common.h"
#include "kernels.h"

// ---------------------------------------------------------------------------
// Embedding gather: x[t, :] = E[tok[t], :] widened to f32.
// "Failed Star / fs — Forward pass → logits", GATHER step (IDs -> residual rows).
__global__ __launch_bounds__(256) void k_embed(const uint16_t* __restrict__ E, const int32_t* __restrict__ tok,
                                               int H, float* __restrict__ x) {
  const int t = blockIdx.x;
  const int id = tok[t];
  const uint16_t* row = E + (size_t)id * H;
  for (int k = threadIdx.x * 4; k < H; k += 256 * 4) {
    u32x2 w = *reinterpret_cast<const u32x2*>(row + k);
    f32x4 o = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    *reinterpret_cast<f32x4*>(x + (size_t)t * H + k) = o;
  }
}

void launch_embed(hipStream_t s, const uint16_t* E, const int32_t* tok, int T, int H, float* x) {
  hipLaunchKernelGGL(k_embed, dim3(T), dim3(256), 0, s, E, tok, H, x);
}

// ---------------------------------------------------------------------------
// Input staging shared by the GEMV kernels: rows [T][K] of the input into LDS,
// optionally RMS-normalised with gains (RMSNorm as a GEMV prologue).
// h[t][k] = x[t][k] * g[k] / sqrt(mean_k x[t][k]^2 + eps)
// Each thread requests up to kStageBatch 16-byte pieces before storing any, so
// a row costs one L2 round trip per 4096 (or 12288) columns, not one per 1024.
constexpr int kStageBatch = 12;

__device__ __forceinline__ void stage_input(const float* __restrict__ x, int ldx, int T, int K,
                                            const float* __restrict__ gain, float eps, float* h, float* red) {
  for (int t = 0; t < T; ++t) {
    const float* xr = x + (size_t)t * ldx;
    float ss = 0.f;
    for (int k0 = 0; k0 < K; k0 += kStageBatch * 1024) {
      f32x4 v[kStageBatch];
#pragma unroll
      for (int i = 0; i < kStageBatch; ++i) {
        const int k = k0 + (threadIdx.x + i * 256) * 4;
        if (k < K) v[i] = *reinterpret_cast<const f32x4*>(xr + k);
      }
#pragma unroll
      for (int i = 0; i < kStageBatch; ++i) {
        const int k = k0 + (threadIdx.x + i * 256) * 4;
        if (k < K) {
          *reinterpret_cast<f32x4*>(h + t * K + k) = v[i];
          ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        }
      }
    }
    if (gain) {  // each thread rescales the pieces it stored
      float tot = block_sum_256(ss, red);
      float r = 1.0f / sqrtf(tot / (float)K + eps);
      for (int k = threadIdx.x * 4; k < K; k += 1024) {
        f32x4 v = *reinterpret_cast<f32x4*>(h + t * K + k);
        f32x4 g = *reinterpret_cast<const f32x4*>(gain + k);
        v = v * r * g;
        *reinterpret_cast<f32x4*>(h + t * K + k) = v;
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// bf16 GEMV / skinny GEMM for T <= GEMV_MAX_T input rows:
//   y[t][n] (=|+=) sum_k W[n][k] * h[t][k] (+ bias[n])
// W row-major [N][K] (the [out, in] layout of the pages).  Each wave owns RPW
// consecutive output rows; each lane streams 16-byte chunks of those rows,
// 512 columns per pass of the wave.  The weights of NP passes are requested
// together (the first NP before the input is staged), so a row of up to
// NP * 512 columns costs one HBM round trip.  The wave-wide sum of a row is
// taken in a fixed order.  TM = 1 (decode) keeps the register count low.
template <int RPW, int TM, int NP>
__global__ __launch_bounds__(256) void k_gemv_bf16(const uint16_t* __restrict__ W, int N, int K,
                                                   const float* __restrict__ x, int ldx, int T,
                                                   const float* __restrict__ gain, float eps,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ y, int ldy, int accumulate) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int np = (K + 511) / 512;
  u32x4 w[NP][RPW];
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = (pb + p) * 512 + lane * 8;
      if (k < K) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int n = min(n0 + i, N - 1);
          w[p][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(W + (size_t)n * K + k));
        }
      }
    }
  };
  if (n0 < N) load(0);
  stage_input(x, ldx, T, K, gain, eps, h, red);
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
      const int k = (pb + p) * 512 + lane * 8;
      if (k < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) acc[i][t] += dot8(w[p][i], h + t * K + k);
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
        float s = wave_sum(acc[i][t]);
        const int n = n0 + i;
        if (lane == 0 && n < N) {
          float* yp = y + (size_t)t * ldy + n;
          float v = s + (bias ? bias[n] : 0.f);
          *yp = accumulate ? (*yp + v) : v;
        }
      }
    }
  }
}

// Rows per wave: as many as max_rpw while the grid (four waves per block)
// still gives every CU at least two blocks.
static int rows_per_wave(int N, int ncu, int max_rpw) {
  int r = max_rpw;
  while (r > 1 && (N + 4 * r - 1) / (4 * r) < 2 * ncu) r >>= 1;
  return r;
}

// Passes requested together: the row's pass count rounded up to 1, 2, 4 or 8.
static int bf16_np(int K) {
  const int np = (K + 511) / 512;
  return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
}

template <int RPW, int NP>
static void gemv_bf16_np(hipStream_t s, const uint16_t* W, int N, int K, const float* x, int ldx, int T,
                         const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate) {
  const dim3 grid((N + 4 * RPW - 1) / (4 * RPW));
  const size_t lds = (8 + (size_t)T * K) * sizeof(float);
  if (T == 1)
    hipLaunchKernelGGL((k_gemv_bf16<RPW, 1, NP>), grid, dim3(256), lds, s, W, N, K, x, ldx, T, gain, eps, bias, y,
                       ldy, accumulate);
  else
    hipLaunchKernelGGL((k_gemv_bf16<RPW, GEMV_MAX_T, 1>), grid, dim3(256), lds, s, W, N, K, x, ldx, T, gain, eps,
                       bias, y, ldy, accumulate);
}

template <int RPW>
static void gemv_bf16_t(hipStream_t s, const uint16_t* W, int N, int K, const float* x, int ldx, int T,
                        const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate) {
  switch (bf16_np(K)) {
    case 1: gemv_bf16_np<RPW, 1>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    case 2: gemv_bf16_np<RPW, 2>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    case 4: gemv_bf16_np<RPW, 4>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    default: gemv_bf16_np<RPW, 8>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
  }
}

void launch_gemv_bf16(hipStream_t s, const uint16_t* W, int N, int K, const float* x, int ldx, int T,
                      const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate, int ncu) {
  switch (rows_per_wave(N, ncu, GEMV_RPW)) {
    case 4: gemv_bf16_t<4>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    case 2: gemv_bf16_t<2>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
    default: gemv_bf16_t<1>(s, W, N, K, x, ldx, T, gain, eps, bias, y, ldy, accumulate); break;
  }
}

// ---------------------------------------------------------------------------
// Fused gate/up GEMV with the SiLU(gate) * up epilogue and an RMSNorm prologue:
//   a[t][i] = SiLU(sum_k Wg[i][k] h[t][k]) * (sum_k Wu[i][k] h[t][k])
// "Failed Star / fs" block figure (SwiGLU); the gated product is formed in
// registers and never stored separately.  Loads are issued as in k_gemv_bf16.
template <int RPW, int TM, int NP>
__global__ __launch_bounds__(256) void k_gemv_gateup_bf16(const uint16_t* __restrict__ Wg,
                                                          const uint16_t* __restrict__ Wu, int N, int K,
                                                          const float* __restrict__ x, int ldx, int T,
                                                          const float* __restrict__ gain, float eps,
                                                          float* __restrict__ a, int lda) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  const int np = (K + 511) / 512;
  u32x4 wg[NP][RPW], wu[NP][RPW];
  auto load = [&](int pb) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int k = (pb + p) * 512 + lane * 8;
      if (k < K) {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int n = min(n0 + i, N - 1);
          wg[p][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wg + (size_t)n * K + k));
          wu[p][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Wu + (size_t)n * K + k));
        }
      }
    }
  };
  if (n0 < N) load(0);
  stage_input(x, ldx, T, K, gain, eps, h, red);
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
      const int k = (pb + p) * 512 + lane * 8;
      if (k < K) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          if (t < T) {
#pragma unroll
            for (int i = 0; i < RPW; ++i) {
              ag[i][t] += dot8(wg[p][i], h + t * K + k);
              au[i][t] += dot8(wu[p][i], h + t * K + k);
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
        float g = wave_sum(ag[i][t]);
        float u = wave_sum(au[i][t]);
        const int n = n0 + i;
        if (lane == 0 && n < N) a[(size_t)t * lda + n] = silu_f(g) * u;
      }
    }
  }
}

template <int RPW, int NP>
static void gateup_bf16_np(hipStream_t s, const uint16_t* Wg, const uint16_t* Wu, int N, int K, const float* x,
                           int ldx, int T, const float* gain, float eps, float* a, int lda) {
  const dim3 grid((N + 4 * RPW - 1) / (4 * RPW));
  const size_t lds = (8 + (size_t)T * K) * sizeof(float);
  if (T == 1)
    hipLaunchKernelGGL((k_gemv_gateup_bf16<RPW, 1, NP>), grid, dim3(256), lds, s, Wg, Wu, N, K, x, ldx, T, gain, eps,
                       a, lda);
  else
    hipLaunchKernelGGL((k_gemv_gateup_bf16<RPW, GEMV_MAX_T, 1>), grid, dim3(256), lds, s, Wg, Wu, N, K, x, ldx, T,
                       gain, eps, a, lda);
}

template <int RPW>
static void gateup_bf16_t(hipStream_t s, const uint16_t* Wg, const uint16_t* Wu, int N, int K, const float* x,
                          int ldx, int T, const float* gain, float eps, float* a, int lda) {
  switch (bf16_np(K)) {
    case 1: gateup_bf16_np<RPW, 1>(s, Wg, Wu, N, K, x, ldx, T, gain, eps, a, lda); break;
    case 2: gateup_bf16_np<RPW, 2>(s, Wg, Wu, N, K, x, ldx, T, gain, eps, a, lda); break;
    default: gateup_bf16_np<RPW, 4>(s, Wg, Wu, N, K, x, ldx, T, gain, eps, a, lda); break;
  }
}

void launch_gemv_gateup_bf16(hipStream_t s, const uint16_t* Wg, const uint16_t* Wu, int N, int K, const float* x,
                             int ldx, int T, const float* gain, float eps, float* a, int lda, int ncu) {
  switch (rows_per_wave(N, ncu, GATEUP_RPW)) {
    case 2: gateup_bf16_t<2>(s, Wg, Wu, N, K, x, ldx, T, gain, eps, a, lda); break;
    default: gateup_bf16_t<1>(s, Wg, Wu, N, K, x, ldx, T, gain, eps, a, lda); break;
  }
}

// ---------------------------------------------------------------------------
// Final RMSNorm + tied LM head for one row, with per-block argmax partials.
//   logits[v] = sum_k E[v][k] * xf[k];  partial[b] = (max logit, lowest id) over the block's rows.
// "Failed Star / fs", LAST ROW step (tied table as the [V, H] output linear).
__global__ __launch_bounds__(256) void k_lmhead_bf16(const uint16_t* __restrict__ E, int V, int H,
                                                     const float* __restrict__ x, const float* __restrict__ gain,
                                                     float eps, float* __restrict__ logits,
                                                     float* __restrict__ part_val, int32_t* __restrict__ part_idx,
                                                     float* __restrict__ xf_out) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  __shared__ float bval[4];
  __shared__ int32_t bidx[4];
  stage_input(x, H, 1, H, gain, eps, h, red);
  if (xf_out && blockIdx.x == 0)
    for (int k = threadIdx.x; k < H; k += 256) xf_out[k] = h[k];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * LMHEAD_RPW;
  float acc[LMHEAD_RPW];
#pragma unroll
  for (int i = 0; i < LMHEAD_RPW; ++i) acc[i] = 0.f;
  if (n0 < V) {
    for (int k = lane * 8; k < H; k += 512) {
      u32x4 w[LMHEAD_RPW];
#pragma unroll
      for (int i = 0; i < LMHEAD_RPW; ++i) {
        const int n = min(n0 + i, V - 1);
        w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(E + (size_t)n * H + k));
      }
#pragma unroll
      for (int i = 0; i < LMHEAD_RPW; ++i) acc[i] += dot8(w[i], h + k);
    }
  }
  float best = -INFINITY;
  int32_t bi = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < LMHEAD_RPW; ++i) {
    float s = wave_sum(acc[i]);
    const int n = n0 + i;
    if (n < V) {
      if (lane == 0) logits[n] = s;
      if (s > best) { best = s; bi = n; }  // rows visited in increasing id: ties keep the lowest
    }
  }
  if (lane == 0) { bval[wave] = best; bidx[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = bval[0];
    int32_t bj = bidx[0];
    for (int w = 1; w < 4; ++w)
      if (bval[w] > bv || (bval[w] == bv && bidx[w] < bj)) { bv = bval[w]; bj = bidx[w]; }
    part_val[blockIdx.x] = bv;
    part_idx[blockIdx.x] = bj;
  }
}

// Streaming form of the LM head (hidden a multiple of 512, HP = hidden / 512):
// a fixed grid of at most 512 workgroups, each staging the normed row once and
// owning RB contiguous vocabulary rows (RB a multiple of 16); wave w takes
// the 4-row chunks w, w + 4, ... of them, the next chunk's rows requested
// while the current one is reduced (rows past the workgroup's range read
// zeros from a bounded buffer record, without memory traffic, so every
// chunk issues the same loads and no wait is forced at a branch).
constexpr int kLmPastRecord = 0x7FFFFFF0;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t lm_record(const void* p, int bytes) {
  const uint64_t v = (uint64_t)p;
  const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <int HP>
__global__ __launch_bounds__(256) void k_lmhead_stream(const uint16_t* __restrict__ E, int V, int H, int RB,
                                                       const float* __restrict__ x, const float* __restrict__ gain,
                                                       float eps, float* __restrict__ logits,
                                                       float* __restrict__ part_val, int32_t* __restrict__ part_idx,
                                                       float* __restrict__ xf_out) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  __shared__ float bval[4];
  __shared__ int32_t bidx[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int base = blockIdx.x * RB, rowend = min(V, base + RB), nrow = max(0, rowend - base);
  const __amdgpu_buffer_rsrc_t re = lm_record(E + (size_t)min(base, V) * H, nrow * H * 2);
  const int nch = RB / 16;  // 4-row chunks per wave
  u32x4 wa[4][HP], wb[4][HP];
  auto load = [&](u32x4 (&w)[4][HP], int j) {
    const int r0 = (wave + 4 * j) * 4;  // first row of the chunk, in the workgroup's range
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int off = r0 + i < nrow ? ((r0 + i) * H + lane * 8) * 2 : kLmPastRecord;
      asm volatile("" : "+v"(off));  // (opaque: one load each, no branch)
#pragma unroll
      for (int p = 0; p < HP; ++p)
        w[i][p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(re, off, p * 1024, 2 /* streamed */));
    }
  };
  if (nch > 0) load(wa, 0);  // requested before the input is staged
  stage_input(x, H, 1, H, gain, eps, h, red);
  if (xf_out && blockIdx.x == 0)
    for (int k = threadIdx.x; k < H; k += 256) xf_out[k] = h[k];
  float best = -INFINITY;
  int32_t bi = 0x7fffffff;
  auto reduce = [&](u32x4 (&w)[4][HP], int j) {
    const int r0 = (wave + 4 * j) * 4;
    float acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = 0.f;
#pragma unroll
      for (int p = 0; p < HP; ++p) acc[i] += dot8(w[i][p], h + p * 512 + lane * 8);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sc = wave_sum(acc[i]);
      if (r0 + i < nrow) {
        const int n = base + r0 + i;
        if (lane == 0) logits[n] = sc;
        if (sc > best) { best = sc; bi = n; }  // rows visited in increasing id: ties keep the lowest
      }
    }
  };
  for (int j = 0; j < nch; j += 2) {  // uniform; chunks j (in wa) and j + 1 (in wb)
    load(wb, j + 1);
    reduce(wa, j);
    load(wa, j + 2);
    reduce(wb, j + 1);
  }
  if (lane == 0) { bval[wave] = best; bidx[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float bv = bval[0];
    int32_t bj = bidx[0];
    for (int w = 1; w < 4; ++w)
      if (bval[w] > bv || (bval[w] == bv && bidx[w] < bj)) { bv = bval[w]; bj = bidx[w]; }
    part_val[blockIdx.x] = bv;
    part_idx[blockIdx.x] = bj;
  }
}

int lmhead_blocks(int V) { return (V + 4 * LMHEAD_RPW - 1) / (4 * LMHEAD_RPW); }

int launch_lmhead_bf16(hipStream_t s, const uint16_t* E, int V, int H, const float* x, const float* gain, float eps,
                       float* logits, float* part_val, int32_t* part_idx, float* xf_out) {
  const size_t lds = (8 + (size_t)H) * sizeof(float);
  const int hp = H / 512;
  if (H % 512 == 0 && (hp == 1 || hp == 2 || hp == 4 || hp == 8) && (size_t)V * H * 2 < ((size_t)1 << 31)) {
    const int grid = std::min(512, (V + 15) / 16);
    const int RB = (V + grid * 16 - 1) / (grid * 16) * 16;
#define QD_LM(HP_)                                                                                                \
  hipLaunchKernelGGL(k_lmhead_stream<HP_>, dim3(grid), dim3(256), lds, s, E, V, H, RB, x, gain, eps, logits,     \
                     part_val, part_idx, xf_out)
    if (hp == 1) QD_LM(1);
    else if (hp == 2) QD_LM(2);
    else if (hp == 4) QD_LM(4);
    else QD_LM(8);
#undef QD_LM
    return grid;
  }
  hipLaunchKernelGGL(k_lmhead_bf16, dim3(lmhead_blocks(V)), dim3(256), lds, s, E, V, H, x, gain, eps, logits, part_val,
                     part_idx, xf_out);
  return lmhead_blocks(V);
}

// ---------------------------------------------------------------------------
// Final greedy choice over the per-block partials (ties -> lowest id), then
// advance the device-resident step state: token := choice, pos += advance, step += 1.
// "flashmoon demo/README.md", Performance notes: argmax stays on the GPU and
// only the token id crosses to the host.
__global__ __launch_bounds__(256) void k_argmax_final(const float* __restrict__ part_val,
                                                      const int32_t* __restrict__ part_idx, int nparts,
                                                      DevState* st, int advance, int32_t* token_out) {
  __shared__ float sv[256];
  __shared__ int32_t si[256];
  float bv = -INFINITY;
  int32_t bj = 0x7fffffff;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    float v = part_val[i];
    int32_t j = part_idx[i];
    if (v > bv || (v == bv && j < bj)) { bv = v; bj = j; }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bj;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      float v = sv[threadIdx.x + off];
      int32_t j = si[threadIdx.x + off];
      if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && j < si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = j;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int32_t tok = si[0];
    if (tok == 0x7fffffff) tok = 0;  // only if every logit was NaN
    st->token = tok;
    st->pos += advance;
    st->step += 1;
    if (token_out) *token_out = tok;
  }
}

void launch_argmax_final(hipStream_t s, const float* part_val, const int32_t* part_idx, int nparts, DevState* st,
                         int advance, int32_t* token_out) {
  hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(256), 0, s, part_val, part_idx, nparts, st, advance, token_out);
}

// ---------------------------------------------------------------------------
// Final RMSNorm + tied LM head for T <= LMHEAD_ROWS rows at once (speculative
// verification): every E row is read once for all T rows, so the bytes of a
// T-row pass are those of one row.  logits[t][v] (t-th row, ld V) and per-block
// argmax partials part_val / part_idx [t][nblk] (lowest id on ties).
__global__ __launch_bounds__(256) void k_lmhead_rows_bf16(const uint16_t* __restrict__ E, int V, int H,
                                                          const float* __restrict__ x, int T,
                                                          const float* __restrict__ gain, float eps,
                                                          float* __restrict__ logits, float* __restrict__ part_val,
                                                          int32_t* __restrict__ part_idx, int nblk) {
  extern __shared__ float smem[];
  float* red = smem;
  float* h = smem + 8;
  __shared__ float bval[LMHEAD_ROWS][4];
  __shared__ int32_t bidx[LMHEAD_ROWS][4];
  stage_input(x, H, T, H, gain, eps, h, red);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + wave) * LMHEAD_RPW;
  float acc[LMHEAD_RPW][LMHEAD_ROWS];
#pragma unroll
  for (int i = 0; i < LMHEAD_RPW; ++i)
#pragma unroll
    for (int t = 0; t < LMHEAD_ROWS; ++t) acc[i][t] = 0.f;
  if (n0 < V) {
    for (int k = lane * 8; k < H; k += 512) {
      u32x4 w[LMHEAD_RPW];
#pragma unroll
      for (int i = 0; i < LMHEAD_RPW; ++i) {
        const int n = min(n0 + i, V - 1);
        w[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(E + (size_t)n * H + k));
      }
#pragma unroll
      for (int t = 0; t < LMHEAD_ROWS; ++t)
        if (t < T) {
#pragma unroll
          for (int i = 0; i < LMHEAD_RPW; ++i) acc[i][t] += dot8(w[i], h + (size_t)t * H + k);
        }
    }
  }
#pragma unroll
  for (int t = 0; t < LMHEAD_ROWS; ++t) {
    if (t >= T) break;
    float best = -INFINITY;
    int32_t bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < LMHEAD_RPW; ++i) {
      const float sv = wave_sum(acc[i][t]);
      const int n = n0 + i;
      if (n < V) {
        if (lane == 0) logits[(size_t)t * V + n] = sv;
        if (sv > best) { best = sv; bi = n; }  // rows visited in increasing id: ties keep the lowest
      }
    }
    if (lane == 0) { bval[t][wave] = best; bidx[t][wave] = bi; }
  }
  __syncthreads();
  if (threadIdx.x < T) {
    const int t = threadIdx.x;
    float bv = bval[t][0];
    int32_t bj = bidx[t][0];
    for (int w = 1; w < 4; ++w)
      if (bval[t][w] > bv || (bval[t][w] == bv && bidx[t][w] < bj)) { bv = bval[t][w]; bj = bidx[t][w]; }
    part_val[(size_t)t * nblk + blockIdx.x] = bv;
    part_idx[(size_t)t * nblk + blockIdx.x] = bj;
  }
}

// Greedy choice of each of T rows from its per-block partials (block t: row
// t), into choice[t]; the block of the last row then advances the step state
// as T decode steps would: token := its choice, pos += T, step += T.
__global__ __launch_bounds__(256) void k_argmax_rows(const float* __restrict__ part_val,
                                                     const int32_t* __restrict__ part_idx, int nblk, int nparts,
                                                     int T, DevState* st, int32_t* __restrict__ choice) {
  __shared__ float sv[256];
  __shared__ int32_t si[256];
  const int t = blockIdx.x;
  float bv = -INFINITY;
  int32_t bj = 0x7fffffff;
  for (int i = threadIdx.x; i < nparts; i += 256) {  // (row t's partials at stride nblk)
    const float v = part_val[(size_t)t * nblk + i];
    const int32_t j = part_idx[(size_t)t * nblk + i];
    if (v > bv || (v == bv && j < bj)) { bv = v; bj = j; }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bj;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      const float v = sv[threadIdx.x + off];
      const int32_t j = si[threadIdx.x + off];
      if (v > sv[threadIdx.x] || (v == sv[threadIdx.x] && j < si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = j;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int32_t tok = si[0];
    if (tok == 0x7fffffff) tok = 0;  // only if every logit was NaN
    choice[t] = tok;
    if (t == T - 1) {
      st->token = tok;
      st->pos += T;
      st->step += T;
    }
  }
}

// Drop the last n positions: pos -= n, step -= n, the next input token set.
__global__ void k_rewind_state(DevState* st, int n, int32_t token) {
  if (threadIdx.x == 0) {
    st->pos -= n;
    st->step = st->step >= n ? st->step - n : 0;
    st->token = token;
  }
}

// The LM head of up to 8 rows on the matrix cores: at most 512 workgroups,
// each staging the rows' final-normed values once as bf16 halves (A rows
// 0-7: hi of rows 0-7, A rows 8-15: lo; rows past T are zeros) and owning RB
// contiguous vocabulary rows (a multiple of 64); wave w takes the 16-row
// chunks w, w + 4, ... of them as the B operand of v_mfma_f32_16x16x32_bf16
// (lane l: vocabulary row l % 16, columns 8 (l / 16) .. + 7 of each 32-column
// K-step), 16 K-steps of loads per group, the next group in flight.  D rows
// t and 8 + t are row t's hi and lo products: added across lanes l, l + 32.
// Each row keeps a running argmax (ties to the lowest id); partials
// part[t][pstride] for the workgroups.
constexpr int kLmKg = 16;  // K-steps per load group
__global__ __launch_bounds__(256) void k_lmhead_rows_mfma(const uint16_t* __restrict__ E, int V, int H, int RB,
                                                          const float* __restrict__ x, int T,
                                                          const float* __restrict__ gain, float eps,
                                                          float* __restrict__ logits, float* __restrict__ part_val,
                                                          int32_t* __restrict__ part_idx, int pstride) {
  extern __shared__ __align__(16) uint16_t sa[];  // [16][H + 8] bf16
  __shared__ float red[4][LMHEAD_ROWS];
  __shared__ float bval[LMHEAD_ROWS][4];
  __shared__ int32_t bidx[LMHEAD_ROWS][4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int LS = H + 8;
  // ---- the rows' RMS scales, then their hi / lo halves into LDS
  float ss[LMHEAD_ROWS];
#pragma unroll
  for (int t = 0; t < LMHEAD_ROWS; ++t) {
    ss[t] = 0.f;
    if (t < T)
      for (int k = tid * 4; k < H; k += 1024) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(x + (size_t)t * H + k);
        ss[t] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    ss[t] = wave_sum(ss[t]);
    if (lane == 0) red[wave][t] = ss[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < LMHEAD_ROWS; ++t) {
    const float r = 1.0f / sqrtf((red[0][t] + red[1][t] + red[2][t] + red[3][t]) / (float)H + eps);
    for (int k = tid * 4; k < H; k += 1024) {
      uint32_t hi[4], lo[4];
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < T) {
        v = *reinterpret_cast<const f32x4*>(x + (size_t)t * H + k) * r;
        if (gain) v = v * *reinterpret_cast<const f32x4*>(gain + k);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hi[i] = bf16_rne(v[i]);
        lo[i] = bf16_rne(v[i] - __uint_as_float(hi[i] << 16));
      }
      *reinterpret_cast<uint2*>(sa + (size_t)t * LS + k) = uint2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
      *reinterpret_cast<uint2*>(sa + (size_t)(8 + t) * LS + k) = uint2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
    }
  }
  __syncthreads();
  // ---- the workgroup's vocabulary rows, 16 per chunk
  const int base = blockIdx.x * RB, rowend = min(V, base + RB), nrow = max(0, rowend - base);
  const __amdgpu_buffer_rsrc_t re = lm_record(E + (size_t)min(base, V) * H, nrow * H * 2);
  const int nl = lane & 15, q = lane >> 4;
  const int ng = H / (32 * kLmKg);          // load groups per chunk
  const int nch = RB / 64;                  // chunks per wave
  const int nu = nch * ng;                  // load groups per wave
  u32x4 bX[kLmKg], bY[kLmKg];
  auto load = [&](u32x4 (&b)[kLmKg], int u) {
    const int j = u / ng, g = u % ng;
    const int row = (wave + 4 * j) * 16 + nl;
    int off = row < nrow && u < nu ? (row * H + g * 32 * kLmKg + 8 * q) * 2 : kLmPastRecord;
    asm volatile("" : "+v"(off));  // (opaque: one load each, no branch)
#pragma unroll
    for (int s2 = 0; s2 < kLmKg; ++s2)
      b[s2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(re, off, s2 * 64, 2 /* streamed */));
  };
  float best[4];
  int32_t bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    best[e] = -INFINITY;
    bi[e] = 0x7fffffff;
  }
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const u32x4 (&b)[kLmKg], int u) {
    const int j = u / ng, g = u % ng;
#pragma unroll
    for (int s2 = 0; s2 < kLmKg; ++s2) {
      const int k = (g * kLmKg + s2) * 32 + 8 * q;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sa + (size_t)nl * LS + k);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b[s2]), acc, 0, 0, 0);
    }
    if (g == ng - 1) {  // uniform: the chunk is done
      const int row = (wave + 4 * j) * 16 + nl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[e]), __float_as_uint(acc[e]), false, false);
        const float v = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // hi + lo products of row 4 q + e
        const int t = 4 * (q & 1) + e;
        if (lane < 32 && t < T && row < nrow) {
          const int n = base + row;
          logits[(size_t)t * V + n] = v;
          if (v > best[e]) { best[e] = v; bi[e] = n; }  // chunks in increasing id: ties keep the lowest
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load(bX, 0);
  for (int u = 0; u < nu; u += 2) {  // uniform
    load(bY, u + 1);
    compute(bX, u);
    load(bX, u + 2);
    if (u + 1 < nu) compute(bY, u + 1);
  }
  // ---- row maxima over the 16 lanes of a row group, then over the waves
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = best[e];
    int32_t id = bi[e];
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const float ov = __shfl_xor(v, m, 64);
      const int32_t oi = __shfl_xor(id, m, 64);
      if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
    }
    const int t = 4 * (q & 1) + e;
    if (lane < 32 && nl == 0 && t < T) {
      bval[t][wave] = v;
      bidx[t][wave] = id;
    }
  }
  __syncthreads();
  if (tid < T) {
    float bv = bval[tid][0];
    int32_t bj = bidx[tid][0];
    for (int w = 1; w < 4; ++w)
      if (bval[tid][w] > bv || (bval[tid][w] == bv && bidx[tid][w] < bj)) { bv = bval[tid][w]; bj = bidx[tid][w]; }
    part_val[(size_t)tid * pstride + blockIdx.x] = bv;
    part_idx[(size_t)tid * pstride + blockIdx.x] = bj;
  }
}

int lmhead_rows_per_pass(int H) {
  int r = (40960 - 8 - 256) / H;  // staged rows (and the block's partials) within 160 KiB of LDS
  if (r > LMHEAD_ROWS) r = LMHEAD_ROWS;
  return r < 1 ? 1 : r;
}

int launch_lmhead_rows_bf16(hipStream_t s, const uint16_t* E, int V, int H, const float* x, int T, const float* gain,
                            float eps, float* logits, float* part_val, int32_t* part_idx) {
  const int nblk = lmhead_blocks(V);
  if (H % (32 * kLmKg) == 0 && H <= 4096 && (size_t)V * H * 2 < ((size_t)1 << 31) && T <= LMHEAD_ROWS) {
    static const bool big_lds = hipFuncSetAttribute((const void*)k_lmhead_rows_mfma,
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    (int)(16 * (4096 + 8) * sizeof(uint16_t))) == hipSuccess;
    (void)big_lds;
    const int grid = std::min(512, (V + 63) / 64);
    const int RB = (V + grid * 64 - 1) / (grid * 64) * 64;
    const size_t lds = (size_t)16 * (H + 8) * sizeof(uint16_t);
    hipLaunchKernelGGL(k_lmhead_rows_mfma, dim3(grid), dim3(256), lds, s, E, V, H, RB, x, T, gain, eps, logits,
                       part_val, part_idx, nblk);
    return grid;
  }
  const size_t lds = (8 + (size_t)T * H) * sizeof(float);
  hipLaunchKernelGGL(k_lmhead_rows_bf16, dim3(nblk), dim3(256), lds, s, E, V, H, x, T, gain, eps, logits, part_val,
                     part_idx, nblk);
  return nblk;
}

void launch_argmax_rows(hipStream_t s, const float* part_val, const int32_t* part_idx, int nblk, int nparts, int T,
                        DevState* st, int32_t* choice) {
  hipLaunchKernelGGL(k_argmax_rows, dim3(T), dim3(256), 0, s, part_val, part_idx, nblk, nparts, T, st, choice);
}

void launch_rewind_state(hipStream_t s, DevState* st, int n, int32_t token) {
  hipLaunchKernelGGL(k_rewind_state, dim3(1), dim3(64), 0, s, st, n, token);
}

// ---------------------------------------------------------------------------
// Per-head QK-RMSNorm, RoPE and the KV-cache write for T rows at positions
// pos .. pos+T-1 (pos read from the device state).
// "flashmoon demo/README.md", decode invariants: RoPE is applied as K is
// written, so the cache holds rotated keys.  The fused projection rows are
// group-major: [kv head g][q heads of g | k_g | v_g].  "Failed Star / fs" block figure:
// QK-norm comes before RoPE.  Pairs are (j, j + d/2).
// grid (T, nq + nkv), block d/2 threads (one per rotation pair).
// The adapter's down products of a batch: u[t][o] = A[o] . (g * x_t / rms(x_t))
// for rows o < n of A (bf16 [n][K]) and input rows t < T (T <= 16).  One
// workgroup per row of A: every thread requests its columns of the A row,
// the gains and every input row at once, then the T dot products and sums
// of squares are reduced together.
constexpr int kLoraDownMaxT = 16;
__global__ __launch_bounds__(256) void k_lora_down_rows(const uint16_t* __restrict__ A, int K,
                                                        const float* __restrict__ x, int ldx, int T,
                                                        const float* __restrict__ gain, float eps,
                                                        float* __restrict__ u, int ldu) {
  __shared__ float red[4][2 * kLoraDownMaxT];
  const int o = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float dot[kLoraDownMaxT], ss[kLoraDownMaxT];
#pragma unroll
  for (int t = 0; t < kLoraDownMaxT; ++t) dot[t] = ss[t] = 0.f;
  for (int c0 = tid * 4; c0 < K; c0 += 1024) {  // 4 columns per thread and pass
    const uint2 a2 = *reinterpret_cast<const uint2*>(A + (size_t)o * K + c0);
    const f32x4 g4 = gain ? *reinterpret_cast<const f32x4*>(gain + c0) : f32x4{1.f, 1.f, 1.f, 1.f};
    const f32x4 ag = f32x4{__uint_as_float(a2.x << 16), __uint_as_float(a2.x & 0xFFFF0000u),
                           __uint_as_float(a2.y << 16), __uint_as_float(a2.y & 0xFFFF0000u)} * g4;
#pragma unroll
    for (int t = 0; t < kLoraDownMaxT; ++t) {
      if (t >= T) break;  // uniform
      const f32x4 v = *reinterpret_cast<const f32x4*>(x + (size_t)t * ldx + c0);
      dot[t] += ag.x * v.x + ag.y * v.y + ag.z * v.z + ag.w * v.w;
      ss[t] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  }
#pragma unroll
  for (int t = 0; t < kLoraDownMaxT; ++t) {
    if (t >= T) break;
    const float dsum = wave_sum(dot[t]), ssum = wave_sum(ss[t]);
    if (lane == 0) {
      red[wave][2 * t] = dsum;
      red[wave][2 * t + 1] = ssum;
    }
  }
  __syncthreads();
  if (tid < T) {
    float dsum = 0.f, ssum = 0.f;
    for (int w = 0; w < 4; ++w) {
      dsum += red[w][2 * tid];
      ssum += red[w][2 * tid + 1];
    }
    u[(size_t)tid * ldu + o] = dsum / sqrtf(ssum / (float)K + eps);
  }
}

// sum_i B[i] u[i] over an adapter row of r bf16 values, in index order.
// Ranks that are multiples of 8 read B in 16-byte and u in 16-byte pieces
// (rows start at multiples of r elements of 16-byte aligned buffers; the
// same fused multiply-adds in the same order).
__device__ __forceinline__ float lora_dot(const uint16_t* __restrict__ B, const float* __restrict__ u, int r) {
  float a = 0.f;
  if ((r & 7) == 0) {
    for (int i = 0; i < r; i += 8) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(B + i);
      const f32x4 u0 = *reinterpret_cast<const f32x4*>(u + i), u1 = *reinterpret_cast<const f32x4*>(u + i + 4);
      a = fmaf(bf16_lo(w.x), u0.x, a);
      a = fmaf(bf16_hi(w.x), u0.y, a);
      a = fmaf(bf16_lo(w.y), u0.z, a);
      a = fmaf(bf16_hi(w.y), u0.w, a);
      a = fmaf(bf16_lo(w.z), u1.x, a);
      a = fmaf(bf16_hi(w.z), u1.y, a);
      a = fmaf(bf16_lo(w.w), u1.z, a);
      a = fmaf(bf16_hi(w.w), u1.w, a);
    }
    return a;
  }
  for (int i = 0; i < r; ++i) a = fmaf(bf16_to_f(B[i]), u[i], a);
  return a;
}

template <typename KVT>
__global__ void k_qk_rope_kv(const float* __restrict__ qkv, int ldqkv, int nq, int nkv, int d,
                             const float* __restrict__ qn, const float* __restrict__ kn, float eps,
                             const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                             const DevState* __restrict__ st, float* __restrict__ q_out,
                             KVT* __restrict__ Kc, KVT* __restrict__ Vc, int max_pos, LoraRows lr) {
  const int t = blockIdx.x, head = blockIdx.y, j = threadIdx.x, half = d >> 1;
  const int pos = st->pos + t;
  const float* row = qkv + (size_t)t * ldqkv;
  const bool is_q = head < nq;
  const int G = nq / nkv;
  const int g = is_q ? head / G : head - nq;  // kv group of this head
  // group-major rows: [kv head g][q heads g*G .. g*G+G-1 | k_g | v_g] x d
  const float* grp = row + (size_t)g * (G + 2) * d;
  const float* src = is_q ? grp + (head % G) * d : grp + G * d;
  float a = src[j], b = src[j + half];
  // adapter (q += s B_q u_q, v += s B_v u_v, before QK-norm and RoPE;
  // "EMBERGLASS (qwen-webgpu-lora) README", LoRA sections)
  const float* ut = lr.u ? lr.u + (size_t)t * lr.ldu : nullptr;
  if (ut && is_q) {
    a += lr.scale * lora_dot(lr.bq + ((size_t)head * d + j) * lr.r, ut, lr.r);
    b += lr.scale * lora_dot(lr.bq + ((size_t)head * d + j + half) * lr.r, ut, lr.r);
  }
  const float* gain = is_q ? qn : kn;
  if (gain) {
    __shared__ float red[4];
    float ss = a * a + b * b;
    ss = wave_sum(ss);
    if (half > 64) {  // more than one wave per head
      if ((j & 63) == 0) red[j >> 6] = ss;
      __syncthreads();
      ss = 0.f;
      for (int w = 0; w < (half + 63) / 64; ++w) ss += red[w];
    }
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    a = a * r * gain[j];
    b = b * r * gain[j + half];
  }
  const float c = cos_t[(size_t)pos * half + j], s = sin_t[(size_t)pos * half + j];
  const float ra = a * c - b * s, rb = b * c + a * s;
  if (is_q) {
    float* qo = q_out + ((size_t)t * nq + head) * d;
    qo[j] = ra;
    qo[j + half] = rb;
  } else {
    KVT* kr = Kc + ((size_t)g * max_pos + pos) * d;
    st_kv(kr + j, ra);
    st_kv(kr + j + half, rb);
    const float* vsrc = grp + (G + 1) * d;
    float va = vsrc[j], vb = vsrc[j + half];
    if (ut) {
      va += lr.scale * lora_dot(lr.bv + ((size_t)g * d + j) * lr.r, ut + lr.r, lr.r);
      vb += lr.scale * lora_dot(lr.bv + ((size_t)g * d + j + half) * lr.r, ut + lr.r, lr.r);
    }
    KVT* vr = Vc + ((size_t)g * max_pos + pos) * d;
    st_kv(vr + j, va);
    st_kv(vr + j + half, vb);
  }
}

void launch_qk_rope_kv(hipStream_t s, const float* qkv, int ldqkv, int T, int nq, int nkv, int d, const float* qn,
                       const float* kn, float eps, const float* cos_t, const float* sin_t, const DevState* st,
                       float* q_out, void* Kc, void* Vc, int max_pos, int kv_bf16, const LoraRows& lr) {
  if (kv_bf16)
    hipLaunchKernelGGL(k_qk_rope_kv<uint16_t>, dim3(T, nq + nkv), dim3(d / 2), 0, s, qkv, ldqkv, nq, nkv, d, qn, kn,
                       eps, cos_t, sin_t, st, q_out, (uint16_t*)Kc, (uint16_t*)Vc, max_pos, lr);
  else
    hipLaunchKernelGGL(k_qk_rope_kv<float>, dim3(T, nq + nkv), dim3(d / 2), 0, s, qkv, ldqkv, nq, nkv, d, qn, kn, eps,
                       cos_t, sin_t, st, q_out, (float*)Kc, (float*)Vc, max_pos, lr);
}

bool launch_lora_down_rows(hipStream_t s, const uint16_t* A, int n, int K, const float* x, int ldx, int T,
                           const float* gain, float eps, float* u, int ldu) {
  if (T < 1 || T > kLoraDownMaxT || K % 1024) return false;
  hipLaunchKernelGGL(k_lora_down_rows, dim3(n), dim3(256), 0, s, A, K, x, ldx, T, gain, eps, u, ldu);
  return true;
}
