// Top-k / temperature / top-p sampling of the next token on the GPU.
//
// "flashmoon demo/README.md — Qwen3-0.6B inference", Quick start and REPL
// commands: temperature 0 is greedy, otherwise temperature, top-k and top-p
// shape the draw; "EMBERGLASS (qwen-webgpu-lora)" notes on decoding: the
// choice stays on the GPU and only the id crosses to the host.  The order of
// the steps is the plain one: keep the top_k logits ordered by (value desc,
// id asc); weights w_i = exp((l_i - l_0) / T); keep the prefix of entries
// whose weight mass before them is < top_p of the total; draw u in [0, 1)
// and take the first kept entry whose running weight exceeds u times the
// kept total.  u comes from SplitMix64 (Steele, Lea and Flood, OOPSLA 2014),
// a counter-based generator: output number (step + 1) from state `seed`,
// top 24 bits over 2^24, with step = tokens chosen since the last reset.
//
// Two kernels after the logits are written:
//   k_topk_block   one wave per slice of 1024 logits: its top-K list, sorted.
//   k_sample_final one wave: K-way merge of the sorted lists (in LDS) into
//                  the global top-K, then the draw; writes the token into the
//                  device step state.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kSlice = 1024;  // logits per k_topk_block wave (16 per lane)
constexpr int kPer = kSlice / 64;
constexpr int kMaxLists = 512;  // lists held per final merge (8 per lane)

// (value desc, id asc): does (v, i) come before (bv, bi)?
__device__ __forceinline__ bool before(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// Wave-wide best (value, id, owner lane) by the order above.
__device__ __forceinline__ void wave_best(float& v, int& i, int& lane_of) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    const int ol = __shfl_xor(lane_of, off, 64);
    if (before(ov, oi, v, i)) {
      v = ov;
      i = oi;
      lane_of = ol;
    }
  }
}

__global__ __launch_bounds__(64) void k_topk_block(const float* __restrict__ logits, int V, int K,
                                                   float* __restrict__ part_val, int32_t* __restrict__ part_idx) {
  const int lane = threadIdx.x, base = blockIdx.x * kSlice;
  float v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int id = base + j * 64 + lane;
    v[j] = id < V ? logits[id] : -INFINITY;
    if (id >= V) taken |= 1u << j;
  }
  for (int r = 0; r < K; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff, bj = -1;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int id = base + j * 64 + lane;
      if (!(taken >> j & 1u) && before(v[j], id, bv, bi)) {
        bv = v[j];
        bi = id;
        bj = j;
      }
    }
    int owner = lane;
    float wv = bv;
    int wi = bi;
    wave_best(wv, wi, owner);
    if (lane == owner && bj >= 0) taken |= 1u << bj;
    if (lane == 0) {
      part_val[(size_t)blockIdx.x * K + r] = wv;
      part_idx[(size_t)blockIdx.x * K + r] = wi;
    }
  }
}

__device__ __forceinline__ uint64_t splitmix64_out(uint64_t seed, uint64_t n) {
  uint64_t z = seed + n * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ __launch_bounds__(64) void k_sample_final(const float* __restrict__ part_val,
                                                     const int32_t* __restrict__ part_idx, int nlists, int K,
                                                     float inv_temp, float top_p, uint64_t seed, DevState* st,
                                                     int32_t* token_out) {
  extern __shared__ float lds[];
  float* lv = lds;                                        // [nlists][K]
  int32_t* li = reinterpret_cast<int32_t*>(lds + nlists * K);  // [nlists][K]
  float* cv = reinterpret_cast<float*>(li + nlists * K);      // [K] merged values
  int32_t* ci = reinterpret_cast<int32_t*>(cv + K);          // [K] merged ids
  const int lane = threadIdx.x;
  for (int i = lane; i < nlists * K; i += 64) {
    lv[i] = part_val[i];
    li[i] = part_idx[i];
  }
  __syncthreads();
  constexpr int kLpl = kMaxLists / 64;  // lists per lane
  int head[kLpl];
#pragma unroll
  for (int j = 0; j < kLpl; ++j) head[j] = 0;
  for (int r = 0; r < K; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff, bj = -1;
#pragma unroll
    for (int j = 0; j < kLpl; ++j) {
      const int b = j * 64 + lane;
      if (b < nlists && head[j] < K) {
        const float v = lv[b * K + head[j]];
        const int id = li[b * K + head[j]];
        if (before(v, id, bv, bi)) {
          bv = v;
          bi = id;
          bj = j;
        }
      }
    }
    int owner = lane;
    float wv = bv;
    int wi = bi;
    wave_best(wv, wi, owner);
    if (lane == owner && bj >= 0) {
#pragma unroll
      for (int j = 0; j < kLpl; ++j)
        if (j == bj) head[j] += 1;
    }
    if (lane == 0) {
      cv[r] = wv;
      ci[r] = wi;
    }
  }
  __syncthreads();
  if (lane != 0) return;
  // weights relative to the best logit; total over the top-K
  float total = 0.f;
  for (int r = 0; r < K; ++r) total += __expf((cv[r] - cv[0]) * inv_temp);
  // kept prefix: entries whose weight mass before them is < top_p of the total
  float kept = 0.f;
  int nkeep = 0;
  for (int r = 0; r < K; ++r) {
    if (r > 0 && !(kept < top_p * total)) break;
    kept += __expf((cv[r] - cv[0]) * inv_temp);
    nkeep = r + 1;
  }
  const int step = st->step - 1;  // the greedy pass that wrote the logits already counted this token
  const float u = (float)(splitmix64_out(seed, (uint64_t)step + 1) >> 40) * (1.0f / 16777216.0f);
  const float target = u * kept;
  float run = 0.f;
  int pick = nkeep - 1;
  for (int r = 0; r < nkeep; ++r) {
    run += __expf((cv[r] - cv[0]) * inv_temp);
    if (target < run) {
      pick = r;
      break;
    }
  }
  int tok = ci[pick];
  if (tok == 0x7fffffff) tok = 0;  // only if every logit was NaN
  st->token = tok;
  if (token_out) *token_out = tok;
}

}  // namespace

int sample_lists(int V) { return (V + kSlice - 1) / kSlice; }

size_t sample_lds_bytes(int V, int K) { return (size_t)sample_lists(V) * K * 8 + (size_t)K * 8; }

bool sample_supported(int V, int K) {
  return K >= 1 && K <= 64 && K <= V && sample_lists(V) <= kMaxLists && sample_lds_bytes(V, K) <= 160 * 1024;
}

int sample_prepare(int V, int K) {
  hipError_t e = hipFuncSetAttribute((const void*)k_sample_final, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)sample_lds_bytes(V, K));
  return e == hipSuccess ? 0 : (int)e;
}

void launch_sample(hipStream_t s, const float* logits, int V, int K, float temperature, float top_p, uint64_t seed,
                   float* part_val, int32_t* part_idx, DevState* st, int32_t* token_out) {
  const int nl = sample_lists(V);
  hipLaunchKernelGGL(k_topk_block, dim3(nl), dim3(64), 0, s, logits, V, K, part_val, part_idx);
  hipLaunchKernelGGL(k_sample_final, dim3(1), dim3(64), sample_lds_bytes(V, K), s, part_val, part_idx, nl, K,
                     1.0f / temperature, top_p, seed, st, token_out);
}
