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

// grid (ceil((nq + nkv) d / 256), min(T, 65535)), block 256: one thread per
// adapted output row (q rows, then v rows), rows of the input strided by gridDim.y.
__global__ __launch_bounds__(256) void k_lora_up(const float* __restrict__ u, int ldu, int T, int r,
                                                 const uint16_t* __restrict__ Bq, const uint16_t* __restrict__ Bv,
                                                 int nq, int nkv, int d, float scale, float* __restrict__ qkv,
                                                 int ldqkv) {
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
  for (int t = blockIdx.y; t < T; t += gridDim.y) {
    const float* ut = u + (size_t)t * ldu + uoff;
    float a = 0.f;
    for (int i = 0; i < r; ++i) a = fmaf(bf16_to_f(B[i]), ut[i], a);
    qkv[(size_t)t * ldqkv + dst] += scale * a;
  }
}

}  // namespace

void launch_lora_up(hipStream_t s, const float* u, int ldu, int T, int r, const uint16_t* Bq, const uint16_t* Bv,
                    int nq, int nkv, int d, float scale, float* qkv, int ldqkv) {
  const dim3 grid(((nq + nkv) * d + 255) / 256, T < 65535 ? T : 65535);
  hipLaunchKernelGGL(k_lora_up, grid, dim3(256), 0, s, u, ldu, T, r, Bq, Bv, nq, nkv, d, scale, qkv, ldqkv);
}
