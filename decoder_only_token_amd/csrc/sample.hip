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
#include <cmath>
#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"
#include "qd.h"

namespace {

constexpr int kSlice = 1024;  // logits per k_topk_block wave (16 per lane)
constexpr int kPer = kSlice / 64;
constexpr int kMaxLists = 512;  // lists held per final merge (8 per lane)
constexpr int kSampleMaxLds = 160 * 1024;  // LDS of one workgroup
constexpr int kMaxDevices = 64;

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
                                                     uint64_t step_arg, int32_t* token_out) {
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
  // with the step state: the greedy pass that wrote the logits already counted this token
  const uint64_t step = st ? (uint64_t)(st->step - 1) : step_arg;
  const float u = (float)(splitmix64_out(seed, step + 1) >> 40) * (1.0f / 16777216.0f);
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
  if (st) st->token = tok;
  if (token_out) *token_out = tok;
}

}  // namespace

int sample_lists(int V) { return (V + kSlice - 1) / kSlice; }

size_t sample_lds_bytes(int V, int K) { return (size_t)sample_lists(V) * K * 8 + (size_t)K * 8; }

bool sample_supported(int V, int K) {
  return K >= 1 && K <= 64 && K <= V && sample_lists(V) <= kMaxLists && sample_lds_bytes(V, K) <= kSampleMaxLds;
}

// The merge kernel's dynamic LDS cap, set to the largest size any supported
// (V, K) needs (or the current device's limit, if lower), so that every
// caller's launch fits.
int sample_prepare() {
  int dev = 0, lim = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)k_sample_final, hipFuncAttributeMaxDynamicSharedMemorySize,
                            lim < kSampleMaxLds ? lim : kSampleMaxLds);
  return e == hipSuccess ? 0 : (int)e;
}

void launch_sample(hipStream_t s, const float* logits, int V, int K, float temperature, float top_p, uint64_t seed,
                   float* part_val, int32_t* part_idx, DevState* st, uint64_t step, int32_t* token_out) {
  const int nl = sample_lists(V);
  hipLaunchKernelGGL(k_topk_block, dim3(nl), dim3(64), 0, s, logits, V, K, part_val, part_idx);
  hipLaunchKernelGGL(k_sample_final, dim3(1), dim3(64), sample_lds_bytes(V, K), s, part_val, part_idx, nl, K,
                     temperature > 0.f ? 1.0f / temperature : 1.0f, top_p, seed, st, step, token_out);
}

// ------------------------------------------------------ handle-free sampling
namespace {

// reason of the last failed handle-free call on this thread
thread_local std::string t_err = "no handle-free call has failed on this thread";

int fail(int code, const char* why) {
  t_err = why;
  return code;
}

// Kernel K of a choice: greedy (no sampling, temperature <= 0, top_k 1) is
// the top-1 list; otherwise top_k after the same checks as the handle's.
int sample_k(const qd_sampling* sp, int V, int* K) {
  if (sp && sp->struct_size != sizeof(qd_sampling)) return fail(QD_E_ABI, "qd_sampling.struct_size mismatch");
  if (sp && !(sp->temperature <= 0.f) && !(sp->temperature > 0.f && std::isfinite(sp->temperature)))
    return fail(QD_E_ARG, "temperature must be finite");
  if (!sp || sp->temperature <= 0.f) {
    *K = 1;
  } else {
    if (sp->top_k < 1 || sp->top_k > 64) return fail(QD_E_ARG, "top_k must be in [1, 64]");
    if (!(sp->top_p > 0.f && sp->top_p <= 1.f)) return fail(QD_E_ARG, "top_p must be in (0, 1]");
    *K = sp->top_k;
  }
  if (V < 1 || !sample_supported(V, *K))
    return fail(QD_E_ARG, "need 1 <= vocab <= 524288, top_k <= vocab and (ceil(vocab / 1024) + 1) * top_k <= 20480");
  return QD_OK;
}

std::mutex g_prep_mu;
bool g_prepared[kMaxDevices];

// Once per device, with that device current: the merge kernel's LDS cap.
int prepare_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices) return fail(QD_E_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> g(g_prep_mu);
  if (!g_prepared[*dev]) {
    if (sample_prepare() != 0) return fail(QD_E_HIP, "hipFuncSetAttribute failed");
    g_prepared[*dev] = true;
  }
  return QD_OK;
}

int launch_checked(const float* logits, int V, int K, const qd_sampling* sp, uint64_t step, int32_t* token,
                   void* ws, hipStream_t s) {
  const size_t lists = (size_t)sample_lists(V) * K;
  float* pv = static_cast<float*>(ws);
  int32_t* pi = reinterpret_cast<int32_t*>(pv + lists);
  const bool draw = K > 1;
  launch_sample(s, logits, V, K, draw ? sp->temperature : 0.f, draw ? sp->top_p : 1.f, draw ? sp->seed : 0, pv, pi,
                nullptr, step, token);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QD_E_HIP, hipGetErrorString(e));
  return QD_OK;
}

}  // namespace

const char* sample_free_error() { return t_err.c_str(); }

// ------------------------------------------- handle-free sampling, no workspace
namespace {

// Scratch of qd_sample_logits_static: the per-slice lists (f32 value, i32
// id) of any supported call, whose lists and merged list fit the merge's
// 160 KiB of LDS, so 160 KiB always suffice; one copy per device, kept until
// the process ends.  Host code never passes
// this name to a kernel (on the host it is only a stand-in): it uses the
// device address that hipGetSymbolAddress returns, per device.
constexpr size_t kStaticScratch = kSampleMaxLds;
__device__ __align__(256) uint8_t scratch[kStaticScratch];

void* g_scratch[kMaxDevices];  // device address of `scratch`, per device (guarded by g_prep_mu)

// Once per device, with that device current: the symbol's device address.
int static_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> g(g_prep_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(QD_E_HIP, "hipGetSymbolAddress(scratch) failed");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return QD_OK;
}

}  // namespace

extern "C" int qd_sample_logits_static(const float* logits_dev, int32_t vocab, const qd_sampling* sampling,
                                       uint64_t step, int32_t* token_dev, void* hip_stream) {
  if (!logits_dev || !token_dev) return fail(QD_E_ARG, "NULL logits or token pointer");
  int K = 0, rc = sample_k(sampling, vocab, &K), dev = 0;
  if (rc != QD_OK) return rc;
  if ((size_t)sample_lists(vocab) * K * 8 > kStaticScratch)
    return fail(QD_E_ARG, "vocab x top_k beyond the static scratch (160 KiB)");
  void* ws = nullptr;
  if ((rc = prepare_device(&dev)) != QD_OK || (rc = static_scratch(dev, &ws)) != QD_OK) return rc;
  return launch_checked(logits_dev, vocab, K, sampling, step, token_dev, ws, static_cast<hipStream_t>(hip_stream));
}

extern "C" {

size_t qd_sample_workspace_bytes(int32_t vocab, const qd_sampling* sampling) {
  int K = 0;
  if (sample_k(sampling, vocab, &K) != QD_OK) return 0;
  return (size_t)sample_lists(vocab) * K * 8;
}

int qd_sample_logits(const float* logits_dev, int32_t vocab, const qd_sampling* sampling, uint64_t step,
                     int32_t* token_dev, void* workspace_dev, size_t workspace_bytes, void* hip_stream) {
  if (!logits_dev || !token_dev || !workspace_dev) return fail(QD_E_ARG, "NULL logits, token or workspace pointer");
  int K = 0, rc = sample_k(sampling, vocab, &K), dev = 0;
  if (rc != QD_OK) return rc;
  if (workspace_bytes < (size_t)sample_lists(vocab) * K * 8)
    return fail(QD_E_ARG, "workspace smaller than qd_sample_workspace_bytes()");
  if ((reinterpret_cast<uintptr_t>(workspace_dev) & 3) != 0) return fail(QD_E_ARG, "workspace not 4-byte aligned");
  if ((rc = prepare_device(&dev)) != QD_OK) return rc;
  return launch_checked(logits_dev, vocab, K, sampling, step, token_dev, workspace_dev,
                        static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
