// Batched prefill projections on the matrix cores of gfx950.
//
// A prompt of T rows makes every projection a dense contraction
// C[T, N] = X[T, K] W[N, K]^T ("Failed Star / fs — Forward pass → logits":
// one [out, in] matrix per projection, applied to every row).  X is f32; W is
// bf16.  X is split into two bf16 halves, X = Xh + Xl (Xh = X rounded to
// bf16, Xl = the rounded remainder), and both are multiplied with W on the
// matrix cores with f32 accumulation, so the product keeps about 16 bits of
// X's mantissa instead of 8.  The RMSNorm of the rows (with its gains) is
// applied before the split.
//
// Tiles: 128 rows of X by 128 output columns per 256-thread block, K in
// steps of 64; each wave owns a 64 x 64 quarter as 4 x 4 tiles of
// v_mfma_f32_16x16x32_bf16.  The K-step tiles of Xh, Xl and W go through
// padded LDS rows (144-byte stride: the 16 rows of a fragment read land on
// distinct banks), and the next K-step is loaded into registers while the
// current one is multiplied.
//
// int4 group-128 weights ("EMBERGLASS (qwen-webgpu-lora) README", "Note on
// weights") go through the same tiles: the 32 codes a thread loads become 32
// exact bf16 integers in the W tile and the matrix cores accumulate code x
// products; the fp16 group scales enter as a running rescale of each output
// column's accumulator (by previous scale / new scale at a group change, by
// the last scale at the end), so no second accumulator set is needed.
#include <hip/hip_fp16.h>

#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDR = BK + 8;  // padded LDS row (bf16): 144 bytes
constexpr int kThreads = 256;

// One block per row: optional RMSNorm with gains, then the hi/lo split.
__global__ __launch_bounds__(256) void k_split_rows(const float* __restrict__ x, int ldx, int K,
                                                    const float* __restrict__ gain, float eps,
                                                    uint16_t* __restrict__ xh, uint16_t* __restrict__ xl) {
  __shared__ float red[8];
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * ldx;
  float r = 1.0f;
  if (gain) {
    float ss = 0.f;
    for (int k = threadIdx.x; k < K; k += 256) ss += xr[k] * xr[k];
    r = 1.0f / sqrtf(block_sum_256(ss, red) / (float)K + eps);
  }
  for (int k = threadIdx.x; k < K; k += 256) {
    const float v = gain ? xr[k] * r * gain[k] : xr[k];
    const uint32_t h = bf16_rne(v);
    const float rest = v - __uint_as_float(h << 16);
    xh[(size_t)t * K + k] = (uint16_t)h;
    xl[(size_t)t * K + k] = (uint16_t)bf16_rne(rest);
  }
}

// The bf16 halves of v (as k_split_rows makes them, without a gain).
__device__ __forceinline__ void store_hilo(uint16_t* __restrict__ h, uint16_t* __restrict__ l, size_t i, float v) {
  const uint32_t hb = bf16_rne(v);
  h[i] = (uint16_t)hb;
  l[i] = (uint16_t)bf16_rne(v - __uint_as_float(hb << 16));
}

enum { EPI_STORE = 0, EPI_ADD = 1, EPI_GATEUP = 2 };

// C tile of block (bm, bn).  EPI_STORE: C = acc (+ bias); EPI_ADD: C += acc;
// EPI_GATEUP: the block's B rows are 64 gate rows and the same 64 up rows,
// C[t][n] = SiLU(gate) * up.
//
// Split-K: with gridDim.z = S > 1, block z multiplies the K range [z Kc,
// (z + 1) Kc) and writes its raw tile to part[z][T][ldp] (ldp = N, or 2 N for
// gate | up); k_splitk_epilogue then sums the S partials in order and applies
// the epilogue.  Small grids (few row tiles times few column tiles) fill the
// GPU this way.
//
// Q4: B / B2 are int4 codes [N][K / 2] with fp16 scales SB / SB2 [N][K / 128]
// (the layout of the int4 GEMVs); Kc is then a multiple of 128.
template <int EPI, bool Q4, int BMT>
__global__ __launch_bounds__(kThreads) void k_gemm_hilo(const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Al,
                                                        int T, int K, const void* __restrict__ B,
                                                        const void* __restrict__ B2, const uint16_t* __restrict__ SB,
                                                        const uint16_t* __restrict__ SB2, int N,
                                                        const float* __restrict__ bias, float* __restrict__ C,
                                                        int ldc, int Kc, float* __restrict__ part,
                                                        uint16_t* __restrict__ Ch, uint16_t* __restrict__ Cl) {
  constexpr int MI = BMT / 32, JA = BMT / 32;  // 16-row tiles per wave, A chunks per thread
  __shared__ __align__(16) uint16_t sA[2][BMT * LDR];  // [hi, lo]
  __shared__ __align__(16) uint16_t sB[BN * LDR];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * BMT;
  const int n0 = blockIdx.y * (EPI == EPI_GATEUP ? BN / 2 : BN);

  // global -> register staging: each tile is BMT (A) or 128 (B) rows x 8
  // chunks of 16 bytes, BMT / 32 or 4 chunks per thread (row = idx / 8,
  // chunk = idx % 8) (an int4 W tile is 128 rows x 32 bytes: one 16-byte load
  // per thread, row = tid / 2, columns 32 (tid % 2) .. + 31)
  constexpr int NB = Q4 ? 1 : 4;
  // two register sets, so that two K-steps' loads are in flight: set X holds
  // A hi / lo, B and (int4, even steps) the 4 group scales of this lane's
  // output columns, requested with the step's tiles
  u32x4 raX[2][JA], rbX[NB], raY[2][JA], rbY[NB];
  uint16_t scX[4], scY[4];
  auto b_row = [&](int row, int& n) -> const void* {
    if (EPI == EPI_GATEUP) {
      n = min(n0 + (row & 63), N - 1);
      return row < 64 ? B : B2;
    }
    n = min(n0 + row, N - 1);
    return B;
  };
  const int kbeg = blockIdx.z * Kc;
  const int nk = min(Kc, K - kbeg) / BK;
  auto gload = [&](u32x4 (&ra)[2][JA], u32x4 (&rb)[NB], uint16_t (&sc)[4], int kt) {
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int idx = tid + j * kThreads, row = idx >> 3, ch = idx & 7;
      const int t = min(m0 + row, T - 1);
      const size_t off = (size_t)t * K + k0 + ch * 8;
      ra[0][j] = *reinterpret_cast<const u32x4*>(Ah + off);
      ra[1][j] = *reinterpret_cast<const u32x4*>(Al + off);
    }
    if (!Q4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + j * kThreads, row = idx >> 3, ch = idx & 7;
        int n;
        const uint16_t* src = static_cast<const uint16_t*>(b_row(row, n));
        rb[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)n * K + k0 + ch * 8));
      }
    } else {
      int n;
      const uint8_t* src = static_cast<const uint8_t*>(b_row(tid >> 1, n));
      rb[0] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(src + (size_t)n * (K / 2) + k0 / 2 + (tid & 1) * 16));
      const int g = k0 / 128;  // (read on every step; used on even ones, where a group starts)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint16_t* S;
        if (EPI == EPI_GATEUP) {
          n = n0 + wn * 32 + (j & 1) * 16 + (lane & 15);
          S = j < 2 ? SB : SB2;
        } else {
          n = n0 + wn * 64 + j * 16 + (lane & 15);
          S = SB;
        }
        sc[j] = S[(size_t)min(n, N - 1) * (K / 128) + g];
      }
    }
  };
  auto sstore = [&](const u32x4 (&ra)[2][JA], const u32x4 (&rb)[NB]) {
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int idx = tid + j * kThreads, row = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(&sA[0][row * LDR + ch * 8]) = ra[0][j];
      *reinterpret_cast<u32x4*>(&sA[1][row * LDR + ch * 8]) = ra[1][j];
    }
    if (!Q4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + j * kThreads, row = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4*>(&sB[row * LDR + ch * 8]) = rb[j];
      }
    } else {
      // byte b of dword m: columns 8 m + 2 b (low nibble) and 8 m + 2 b + 1
      // (high nibble), each code + 8; bf16 of a small integer is exact
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w = rb[0][m];
        u32x4 o;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float f0 = (float)((w >> (8 * b)) & 0xFu) - 8.0f;
          const float f1 = (float)((w >> (8 * b + 4)) & 0xFu) - 8.0f;
          o[b] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
        }
        *reinterpret_cast<u32x4*>(&sB[(tid >> 1) * LDR + (tid & 1) * 32 + m * 8]) = o;
      }
    }
  };

  // Q4: acc holds sum_groups code.x * e_g / e_cur, where e_g is the group's
  // scale (a zero scale keeps the previous one: its codes are all zero);
  // entering a group multiplies acc by e_prev / e_new, and the end by e_last.
  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B rows of this wave's 4 column tiles
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = EPI == EPI_GATEUP ? (j < 2 ? 0 : 64) + wn * 32 + (j & 1) * 16 : wn * 64 + j * 16;

  float scl[4] = {1.f, 1.f, 1.f, 1.f};  // Q4: current scale e of this lane's 4 output columns
  // one K-step from the tiles in LDS (scales of its register set)
  auto step = [&](int kt, const uint16_t (&sc)[4]) {
    if (Q4 && (kt & 1) == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = __half2float(__ushort_as_half(sc[j]));
        if (e > 0.f) {
          const float r = scl[j] / e;
#pragma unroll
          for (int i = 0; i < MI; ++i) acc[i][j] *= r;
          scl[j] = e;
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      // fragments: lane holds row (lane % 16), k = kk + (lane / 16) * 8 .. + 8
      const int fr = lane & 15, fk = kk + (lane >> 4) * 8;
      bf16x8 bh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bh[j] = *reinterpret_cast<const bf16x8*>(&sB[(brow[j] + fr) * LDR + fk]);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int ar = wm * (BMT / 2) + i * 16 + fr;
        const bf16x8 a_hi = *reinterpret_cast<const bf16x8*>(&sA[0][ar * LDR + fk]);
        const bf16x8 a_lo = *reinterpret_cast<const bf16x8*>(&sA[1][ar * LDR + fk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, bh[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, bh[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (BMT == 128) {
    // the 128-row tile (long batches, many workgroups): one register set,
    // the next K-step in flight during this one (a second set would cost
    // occupancy)
    gload(raX, rbX, scX, 0);
    sstore(raX, rbX);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {  // uniform
      uint16_t scc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) scc[j] = scX[j];
      if (kt + 1 < nk) gload(raX, rbX, scX, kt + 1);
      step(kt, scc);
      if (kt + 1 < nk) {
        __syncthreads();  // every wave is done with this K-step's tiles
        sstore(raX, rbX);
        __syncthreads();
      }
    }
  } else {
    // K-steps: step kt computes from LDS while the registers of steps kt + 1
    // and kt + 2 are in flight.  The steady part issues the same loads in every
    // pass (no load under a branch, so no wait for a later load is forced);
    // the last (up to three) steps follow.  (With one step, set Y re-reads it.)
    gload(raX, rbX, scX, 0);
    sstore(raX, rbX);
    __syncthreads();
    uint16_t sc0[4];
  #pragma unroll
    for (int j = 0; j < 4; ++j) sc0[j] = scX[j];
    gload(raY, rbY, scY, min(1, nk - 1));
    int kt = 0;
    for (; kt + 3 < nk; kt += 2) {  // uniform
      uint16_t scc[4];
  #pragma unroll
      for (int j = 0; j < 4; ++j) scc[j] = kt == 0 ? sc0[j] : scX[j];
      gload(raX, rbX, scX, kt + 2);
      step(kt, scc);
      __syncthreads();  // every wave is done with step kt's tiles
      sstore(raY, rbY);
      __syncthreads();
      uint16_t scn[4];
  #pragma unroll
      for (int j = 0; j < 4; ++j) scn[j] = scY[j];
      gload(raY, rbY, scY, kt + 3);
      step(kt + 1, scn);
      __syncthreads();
      sstore(raX, rbX);
      __syncthreads();
    }
    // the tail: step kt in LDS (its scales: sc0 at kt = 0, else set X's),
    // kt + 1 in set Y when it exists, kt + 2 not requested yet
    {
      uint16_t scc[4];
  #pragma unroll
      for (int j = 0; j < 4; ++j) scc[j] = kt == 0 ? sc0[j] : scX[j];
      if (kt + 2 < nk) gload(raX, rbX, scX, kt + 2);
      step(kt, scc);
      if (kt + 1 < nk) {
        __syncthreads();
        sstore(raY, rbY);
        __syncthreads();
        step(kt + 1, scY);
      }
      if (kt + 2 < nk) {
        __syncthreads();
        sstore(raX, rbX);
        __syncthreads();
        step(kt + 2, scX);
      }
    }
  }
  if (Q4) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] *= scl[j];
  }

  // epilogue: acc[i][j] element e of lane is C[row 4 (lane / 16) + e][col lane % 16]
  // of the (i, j) 16 x 16 tile
  if (gridDim.z > 1) {
    const int ldp = EPI == EPI_GATEUP ? 2 * N : N;
    float* P = part + (size_t)blockIdx.z * T * ldp;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = m0 + wm * (BMT / 2) + i * 16 + (lane >> 4) * 4 + e;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int n;
          if (EPI == EPI_GATEUP) {
            n = n0 + wn * 32 + (j & 1) * 16 + (lane & 15);
            if (n < N) P[(size_t)t * ldp + (j < 2 ? 0 : N) + n] = acc[i][j][e];
          } else {
            n = n0 + wn * 64 + j * 16 + (lane & 15);
            if (n < N) P[(size_t)t * ldp + n] = acc[i][j][e];
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = m0 + wm * (BMT / 2) + i * 16 + (lane >> 4) * 4 + e;
      if (t >= T) continue;
      if (EPI == EPI_GATEUP) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 32 + j * 16 + (lane & 15);
          if (n < N) {
            const float g = acc[i][j][e], u = acc[i][j + 2][e];
            const float v = silu_f(g) * u;
            C[(size_t)t * ldc + n] = v;
            if (Ch) store_hilo(Ch, Cl, (size_t)t * ldc + n, v);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          if (n < N) {
            float* cp = C + (size_t)t * ldc + n;
            if (EPI == EPI_ADD) {
              *cp += acc[i][j][e];
            } else {
              *cp = acc[i][j][e] + (bias ? bias[n] : 0.f);
            }
          }
        }
      }
    }
  }
}

// Sum of the S split partials in split order, then the epilogue.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_epilogue(const float* __restrict__ part, int S, int T, int N,
                                                         const float* __restrict__ bias, float* __restrict__ C,
                                                         int ldc, uint16_t* __restrict__ Ch,
                                                         uint16_t* __restrict__ Cl) {
  const size_t total = (size_t)T * N;
  const int ldp = EPI == EPI_GATEUP ? 2 * N : N;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int t = (int)(i / N), n = (int)(i % N);
    float a = 0.f, b = 0.f;
    for (int z = 0; z < S; ++z) {
      const float* P = part + (size_t)z * T * ldp + (size_t)t * ldp;
      a += P[n];
      if (EPI == EPI_GATEUP) b += P[N + n];
    }
    float* cp = C + (size_t)t * ldc + n;
    if (EPI == EPI_GATEUP) {
      const float v = silu_f(a) * b;
      *cp = v;
      if (Ch) store_hilo(Ch, Cl, (size_t)t * ldc + n, v);
    } else if (EPI == EPI_ADD) {
      *cp += a;
    } else {
      *cp = a + (bias ? bias[n] : 0.f);
    }
  }
}

// Row tile of a T-row product: 64 rows for short batches (twice the
// workgroups, so fewer K splits), 128 otherwise.
int gemm_bm(int T) { return T <= 2048 ? 64 : BM; }

// K splits for a T x N product: none when the tiles give every CU a
// workgroup, else enough to do so, each split at least two K-steps long, at
// most 8 splits.
int splits_for(int T, int K, int N, int epi, int ncu) {
  const int bm = gemm_bm(T);
  const int tiles = ((T + bm - 1) / bm) * (epi == EPI_GATEUP ? (N + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN);
  if (tiles >= ncu) return 1;
  int s = (ncu + tiles - 1) / tiles;
  s = std::min(s, std::max(1, K / BK / 2));
  return std::max(1, std::min(s, 8));
}

}  // namespace

bool gemm_supported(int K) { return K % BK == 0; }

size_t gemm_workspace_floats(int T, int K, int N, int ncu) {
  size_t best = 0;
  for (int epi : {EPI_STORE, EPI_GATEUP}) {
    const int s = splits_for(T, K, N, epi, ncu);
    if (s > 1) best = std::max(best, (size_t)s * T * (epi == EPI_GATEUP ? 2 * N : N));
  }
  return best;
}

void launch_split_rows(hipStream_t s, const float* x, int ldx, int T, int K, const float* gain, float eps,
                       uint16_t* xh, uint16_t* xl) {
  hipLaunchKernelGGL(k_split_rows, dim3(T), dim3(256), 0, s, x, ldx, K, gain, eps, xh, xl);
}

namespace {

template <bool Q4>
void launch_gemm(hipStream_t s, int epi, const uint16_t* xh, const uint16_t* xl, int T, int K, const void* W,
                 const void* W2, const uint16_t* SW, const uint16_t* SW2, int N, const float* bias, float* C, int ldc,
                 float* ws, size_t ws_floats, int ncu, uint16_t* ch, uint16_t* cl) {
  int S = splits_for(T, K, N, epi, ncu);
  if ((size_t)S * T * (epi == EPI_GATEUP ? 2 * N : N) > ws_floats || !ws) S = 1;
  const int step = Q4 ? 128 : BK;  // an int4 split holds whole groups
  const int Kc = (K / step + S - 1) / S * step;
  S = (K + Kc - 1) / Kc;  // every split holds at least one K-step
  const int bm = gemm_bm(T);
  const dim3 grid((T + bm - 1) / bm, epi == EPI_GATEUP ? (N + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN, S);
#define QD_GEMM(EPI_, BM_)                                                                                          \
  hipLaunchKernelGGL((k_gemm_hilo<EPI_, Q4, BM_>), grid, dim3(kThreads), 0, s, xh, xl, T, K, W, W2, SW, SW2, N, bias, \
                     C, ldc, Kc, ws, ch, cl)
  switch (epi) {
    case EPI_STORE:
      if (bm == 64) QD_GEMM(EPI_STORE, 64);
      else QD_GEMM(EPI_STORE, BM);
      break;
    case EPI_ADD:
      if (bm == 64) QD_GEMM(EPI_ADD, 64);
      else QD_GEMM(EPI_ADD, BM);
      break;
    default:
      if (bm == 64) QD_GEMM(EPI_GATEUP, 64);
      else QD_GEMM(EPI_GATEUP, BM);
      break;
  }
#undef QD_GEMM
  if (S == 1) return;
  const int blocks = (int)std::min<size_t>(((size_t)T * N + 255) / 256, 4096);
  switch (epi) {
    case EPI_STORE:
      hipLaunchKernelGGL(k_splitk_epilogue<EPI_STORE>, dim3(blocks), dim3(256), 0, s, ws, S, T, N, bias, C, ldc, ch, cl);
      break;
    case EPI_ADD:
      hipLaunchKernelGGL(k_splitk_epilogue<EPI_ADD>, dim3(blocks), dim3(256), 0, s, ws, S, T, N, bias, C, ldc, ch, cl);
      break;
    default:
      hipLaunchKernelGGL(k_splitk_epilogue<EPI_GATEUP>, dim3(blocks), dim3(256), 0, s, ws, S, T, N, bias, C, ldc, ch, cl);
      break;
  }
}

}  // namespace

void launch_gemm_hilo(hipStream_t s, int epi, const uint16_t* xh, const uint16_t* xl, int T, int K, const uint16_t* W,
                      const uint16_t* W2, int N, const float* bias, float* C, int ldc, float* ws, size_t ws_floats,
                      int ncu, uint16_t* ch, uint16_t* cl) {
  launch_gemm<false>(s, epi, xh, xl, T, K, W, W2, nullptr, nullptr, N, bias, C, ldc, ws, ws_floats, ncu, ch, cl);
}

void launch_gemm_q4(hipStream_t s, int epi, const uint16_t* xh, const uint16_t* xl, int T, int K, const uint8_t* W,
                    const uint16_t* SW, const uint8_t* W2, const uint16_t* SW2, int N, const float* bias, float* C,
                    int ldc, float* ws, size_t ws_floats, int ncu, uint16_t* ch, uint16_t* cl) {
  launch_gemm<true>(s, epi, xh, xl, T, K, W, W2, SW, SW2, N, bias, C, ldc, ws, ws_floats, ncu, ch, cl);
}
