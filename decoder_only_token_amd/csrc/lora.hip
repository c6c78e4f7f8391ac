// Low-rank adapter on the q and v projections, as a separate pair of thin
// products after the QKV projection.
//
// "EMBERGLASS (qwen-webgpu-lora) README", LoRA sections: a rank-r adapter is
// applied live to q_proj and v_proj, and clearing it gives the base model back
// exactly.  With h the attention-normed input row,
//   q += (alpha / r) B_q (A_q h),   v += (alpha / r) B_v (A_v h).
// The down products u = [A_q; A_v] h (2 r values per row) come from the
// library's GEMV or matrix-core GEMM over the stacked [2 r, H] matrix; this
// file adds the up products into the fused q|k|v rows.  When no adapter is
// set none of this runs, so the base path is unchanged bit for bit.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kRowsPerBlock = 32;  // input rows per block of the up product
constexpr int kMaxRank = 64;

// grid (ceil((nq + nkv) d / 256), ceil(T / kRowsPerBlock)), block 256: one
// thread per adapted output row (q rows, then v rows) holding its row of B in
// registers; the block's input rows of u are staged in LDS.
__global__ __launch_bounds__(256) void k_lora_up(const float* __restrict__ u, int ldu, int T, int r,
                                                 const uint16_t* __restrict__ Bq, const uint16_t* __restrict__ Bv,
                                                 int nq, int nkv, int d, float scale, float* __restrict__ qkv,
                                                 int ldqkv) {
  __shared__ float us[kRowsPerBlock * 2 * kMaxRank];
  const int t0 = blockIdx.y * kRowsPerBlock, nt = min(kRowsPerBlock, T - t0);
  for (int i = threadIdx.x; i < nt * 2 * r; i += 256) us[i] = u[(size_t)(t0 + i / (2 * r)) * ldu + i % (2 * r)];
  __syncthreads();
  const int row = blockIdx.x * 256 + threadIdx.x;
  const int G = nq / nkv;
  if (row >= (nq + nkv) * d) return;
  const uint16_t* B;
  int uoff, dst;
  if (row < nq * d) {
    const int hq = row / d, j = row % d;
    B = Bq + (size_t)row * r;
    uoff = 0;
    dst = (hq / G) * (G + 2) * d + (hq % G) * d + j;
  } else {
    const int rv = row - nq * d, g = rv / d, j = rv % d;
    B = Bv + (size_t)rv * r;
    uoff = r;
    dst = g * (G + 2) * d + (G + 1) * d + j;
  }
  float b[kMaxRank];
#pragma unroll
  for (int i = 0; i < kMaxRank; ++i) b[i] = i < r ? bf16_to_f(B[i]) : 0.f;
  for (int t = 0; t < nt; ++t) {
    const float* ut = us + t * 2 * r + uoff;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxRank; ++i)
      if (i < r) a = fmaf(b[i], ut[i], a);
    qkv[(size_t)(t0 + t) * ldqkv + dst] += scale * a;
  }
}

}  // namespace

void launch_lora_up(hipStream_t s, const float* u, int ldu, int T, int r, const uint16_t* Bq, const uint16_t* Bv,
                    int nq, int nkv, int d, float scale, float* qkv, int ldqkv) {
  const dim3 grid(((nq + nkv) * d + 255) / 256, (T + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(k_lora_up, grid, dim3(256), 0, s, u, ldu, T, r, Bq, Bv, nq, nkv, d, scale, qkv, ldqkv);
}
