// Persistent decode step for gfx950: the whole single-token forward in ONE
// cooperative kernel launch, one 512-thread workgroup per CU.
//
// A decode step is a chain of ~5 dependent phases per layer.  As separate
// kernels, every dependency costs a launch gap plus the ramp and tail of the
// next kernel.  Here each dependency is a device-scope handshake instead:
// producers publish every value as a 64-bit word {f32 value | tag << 32} with
// one relaxed agent-scope store, and consumers spin with relaxed agent-scope
// loads until every word carries the tag they expect.  No fences, no shared
// counters, no L2 writeback/invalidate: the tag itself says the value is
// there.  Every phase issues its weight (or KV-cache) loads BEFORE it waits
// for its input, so the HBM stream overlaps the handshake latency.
//
// Phases of layer l (tag = seq << 8 | l unless noted):
//   A  rows of q|k|v = W_qkv RMSNorm(x0) + b                     -> QKV
//   B  attention item (kv head g, split s): QK-norm, RoPE, KV-cache
//      write, online softmax over its positions -> partial; the split
//      partials of each head are merged in split order              -> O
//   C  rows of x1 = x0 + W_o o                                     -> X1
//   D1 rows of act = SiLU(W_g h2) * (W_u h2), h2 = RMSNorm(x1)      -> ACT
//   D2 rows of x0' = x1 + W_d act                                  -> X0 (tag l+1)
// then the final RMSNorm + tied LM head with per-CU argmax partials, and the
// argmax over the partials by CU 0, which advances the step state.
//
// Reusing a buffer across layers is safe because every reader of a buffer
// instance is, through the dataflow, a required producer of what the next
// writer of that buffer waits for.
#include "common.h"
#include "persist.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kSeg = 512;  // bf16 per segment: 64 lanes x 8 values (16 bytes each)
constexpr int kBatch = 8;  // segments per wave per load batch
constexpr int D = 128;     // head_dim
constexpr uint64_t kTimeoutTicks = 20000000ull;  // 200 ms of the 100 MHz real-time counter

// Explicit address spaces: without them pointers read from the parameter block
// stay generic and every access becomes a FLAT instruction, which also counts
// against the LDS wait counter, so any LDS wait would drain the weight
// prefetches.  AS1 = global memory, AS4 = constant (uniform, scalar loads).
#define AS1 __attribute__((address_space(1)))
#define AS4 __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ AS1 T* gl(T* p) {
  return (AS1 T*)p;
}

__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(gl(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tagged(uint64_t* p, float v, uint32_t tag) {
  __hip_atomic_store(gl(p), ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(gl(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(gl(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 ld_w16(const uint16_t* p) {  // 8 bf16 weights, streamed once
  return __builtin_nontemporal_load(gl(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ f32x4 ld_f4(const float* p) { return *gl(reinterpret_cast<const f32x4*>(p)); }
__device__ __forceinline__ float ld_f(const float* p) { return *gl(p); }
__device__ __forceinline__ void st_f(float* p, float v) { *gl(p) = v; }
__device__ __forceinline__ uint32_t tag_of(uint32_t seq, int l) { return (seq << 8) | (uint32_t)l; }

// Optional phase trace: slot 0 = kernel start, then (input ready, outputs written)
// for phase p at slots 1 + 2p and 2 + 2p.  Thread 0 of each CU writes.
__device__ __forceinline__ void stamp(const AS4 PersistConst* a, int slot) {
  if (a->trace && threadIdx.x == 0)
    *gl(a->trace + (size_t)blockIdx.x * persist_trace_slots(a->L) + slot) = __builtin_amdgcn_s_memrealtime();
}

struct Smem {
  float vec[16384];             // input vector of the current phase (+ residual rows)
  float part[1024];             // per-(row, wave) partial sums
  float red[16];                // block reductions
  float att[kWaves * 8 * 130];  // per-wave attention states
  float qk[10 * D];             // q heads, k, v of one kv group
  int abort_flag;
};

struct Ctx {
  const AS4 PersistConst* a;
  int pos, S, chunk;
  uint32_t seq;
  uint64_t t0;
  int* abort_lds;
};

struct Seg {
  const uint64_t* src;
  int n;
  float* dst;
};

// Block-collective wait for up to NS segments of tagged values; copies the
// values into LDS once every tag matches.  Returns false block-uniformly on a
// timeout or when another CU has abandoned the step.
template <int NS>
__device__ __forceinline__ bool wait_segs(Ctx& c, const Seg (&sg)[NS], uint32_t tag) {
  constexpr int E = 8;  // values per thread per pass
  int total = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) total += sg[i].n;
  bool ok = !*c.abort_lds;
  for (int base = 0; base < total && ok; base += E * kThreads) {
    uint64_t v[E];
    uint32_t spin = 0;
    for (;;) {
      bool done = true;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int i = base + e * kThreads + threadIdx.x;
        v[e] = (uint64_t)tag << 32;
        if (i < total) {
#pragma unroll
          for (int q = 0; q < NS; ++q) {
            if (i >= 0 && i < sg[q].n) v[e] = ld_tagged(sg[q].src + i);
            i -= sg[q].n;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) done &= (uint32_t)(v[e] >> 32) == tag;
      if (done) break;
      if ((++spin & 31) == 0 &&
          (ld_u32(&c.a->err[0]) != 0 || __builtin_amdgcn_s_memrealtime() - c.t0 > kTimeoutTicks)) {
        st_u32(&c.a->err[0], 1);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (ok) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        int i = base + e * kThreads + threadIdx.x;
        if (i < total) {
#pragma unroll
          for (int q = 0; q < NS; ++q) {
            if (i >= 0 && i < sg[q].n) sg[q].dst[i] = __uint_as_float((uint32_t)v[e]);
            i -= sg[q].n;
          }
        }
      }
    }
  }
  if (!ok) *c.abort_lds = 1;
  __syncthreads();
  return !*c.abort_lds;
}

__device__ __forceinline__ bool wait_vec(Ctx& c, const uint64_t* src, int n, uint32_t tag, float* dst) {
  Seg s[1] = {{src, n, dst}};
  return wait_segs<1>(c, s, tag);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  __syncthreads();
  return t;
}

// In-place RMSNorm of an LDS vector: h[k] = h[k] * g[k] / sqrt(mean(h^2) + eps).
__device__ __forceinline__ void norm_lds(float* h, int K, const float* __restrict__ g, float eps, float* red) {
  float ss = 0.f;
  for (int k = threadIdx.x; k < K; k += kThreads) ss += h[k] * h[k];
  const float r = 1.0f / sqrtf(block_sum(ss, red) / (float)K + eps);
  for (int k = threadIdx.x; k < K; k += kThreads) h[k] = h[k] * r * ld_f(g + k);
  __syncthreads();
}

// rows [r0, r1) of N split evenly over the grid
__device__ __forceinline__ void cu_rows(int N, int& r0, int& r1) {
  r0 = (int)((long)N * blockIdx.x / gridDim.x);
  r1 = (int)((long)N * (blockIdx.x + 1) / gridDim.x);
}

// ---------------------------------------------------------------------------
// Segmented GEMV over the rows this CU owns.  Row v (a virtual row index, so
// gate/up can interleave two matrices) is cut into ceil(K/512) segments; the
// CU's row-major segment list is split into 8 contiguous per-wave ranges.  A
// wave issues its loads in batches of 8 segments; the first batch is issued
// before the phase waits for its input.  A row's partial sum from one wave is
// stored in part[row * 8 + wave]; row totals add the 8 waves in order.
struct SegPlan {
  int K, nseg, s0, s1;
};

__device__ __forceinline__ SegPlan seg_plan(int nrows, int K) {
  SegPlan p;
  p.K = K;
  p.nseg = (K + kSeg - 1) / kSeg;
  const int total = nrows * p.nseg, w = threadIdx.x >> 6;
  p.s0 = (int)((long)total * w / kWaves);
  p.s1 = (int)((long)total * (w + 1) / kWaves);
  return p;
}

template <typename RowFn>
__device__ __forceinline__ void seg_load(const SegPlan& p, int b0, u32x4 (&w)[kBatch], RowFn row) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int s = b0 + i;
    const int r = s / p.nseg, k = (s % p.nseg) * kSeg + lane * 8;
    if (s < p.s1 && k < p.K) w[i] = ld_w16(row(r) + k);
  }
}

__device__ __forceinline__ void seg_compute(const SegPlan& p, int b0, const u32x4 (&w)[kBatch], const float* h,
                                            float& acc, float* part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    const int s = b0 + i;
    if (s < p.s1) {
      const int r = s / p.nseg, k = (s % p.nseg) * kSeg + lane * 8;
      if (k < p.K) acc += dot8(w[i], h + k);
      if (s + 1 == p.s1 || (s + 1) % p.nseg == 0) {  // last segment of this row in this wave
        const float t = wave_sum(acc);
        if (lane == 0) part[r * kWaves + wave] = t;
        acc = 0.f;
      }
    }
  }
}

template <typename RowFn>
__device__ void seg_run(const SegPlan& p, u32x4 (&w0)[kBatch], const float* h, float* part, RowFn row) {
  u32x4 w1[kBatch];
  float acc = 0.f;
  for (int b0 = p.s0; b0 < p.s1; b0 += 2 * kBatch) {
    if (b0 + kBatch < p.s1) seg_load(p, b0 + kBatch, w1, row);
    seg_compute(p, b0, w0, h, acc, part);
    if (b0 + 2 * kBatch < p.s1) seg_load(p, b0 + 2 * kBatch, w0, row);
    if (b0 + kBatch < p.s1) seg_compute(p, b0 + kBatch, w1, h, acc, part);
  }
}

__device__ __forceinline__ void zero_part(float* part, int nrows) {
  for (int i = threadIdx.x; i < nrows * kWaves; i += kThreads) part[i] = 0.f;
}

__device__ __forceinline__ float row_total(const float* part, int r) {
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += part[r * kWaves + w];
  return t;
}

// ---------------------------------------------------------------------------
// Phase A: rows of q|k|v = W_qkv RMSNorm(x0) (+ bias).  Layer 0 reads x0 = E[token].
__device__ __forceinline__ bool phase_qkv(Ctx& c, Smem& sm, int l, const uint16_t* emb) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  int r0, r1;
  cu_rows(a.nqkv, r0, r1);
  const int H = a.H;
  const SegPlan p = seg_plan(r1 - r0, H);
  const uint16_t* W = L.wqkv + (size_t)r0 * H;
  auto row = [&](int r) { return W + (size_t)r * H; };
  u32x4 w0[kBatch];
  seg_load(p, p.s0, w0, row);
  zero_part(sm.part, r1 - r0);
  if (l == 0) {
    for (int k = threadIdx.x; k < H; k += kThreads) sm.vec[k] = bf16_to_f(*gl(emb + k));
    __syncthreads();
  } else if (!wait_vec(c, a.X0, H, tag_of(c.seq, l), sm.vec)) {
    return false;
  }
  norm_lds(sm.vec, H, L.attn_norm, a.eps, sm.red);
  stamp(c.a, 1 + 2 * (5 * l));
  seg_run(p, w0, sm.vec, sm.part, row);
  __syncthreads();
  const uint32_t tag = tag_of(c.seq, l);
  for (int r = threadIdx.x; r < r1 - r0; r += kThreads) {
    float v = row_total(sm.part, r);
    if (L.bqkv) v += ld_f(L.bqkv + r0 + r);
    st_tagged(a.QKV + r0 + r, v, tag);
  }
  stamp(c.a, 2 + 2 * (5 * l));
  return true;
}

// Phase B: attention item (kv head g, split s) of the grid; items >= nkv * S idle.
template <int G>
__device__ __forceinline__ bool phase_attn(Ctx& c, Smem& sm, int l) {
  constexpr int NP = 4;  // positions per half-wave held in registers per batch
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  const int S = c.S, pos = c.pos, ctx = pos + 1;
  if ((int)blockIdx.x >= a.nkv * S) return true;
  const int g = blockIdx.x / S, s = blockIdx.x % S;
  const int p_begin = s * c.chunk, p_end = min(p_begin + c.chunk, ctx);
  const uint32_t tag = tag_of(c.seq, l);
  const int hw = threadIdx.x >> 5, sub = threadIdx.x & 31;  // 16 half-waves
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* Kg = a.Kc + ((size_t)l * a.nkv + g) * a.max_pos * D;
  float* Vg = a.Vc + ((size_t)l * a.nkv + g) * a.max_pos * D;
  // 1. prefetch cached K/V of this half-wave's first positions (not the new one)
  f32x4 kr[NP], vr[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int p = p_begin + hw + 16 * i;
    if (p < p_end && p != pos) {
      kr[i] = ld_f4(Kg + (size_t)p * D + sub * 4);
      vr[i] = ld_f4(Vg + (size_t)p * D + sub * 4);
    }
  }
  // 2. wait for this group's q heads, k and v
  float* qk = sm.qk;  // [G q heads][k][v] x 128
  {
    Seg sg[3] = {{a.QKV + g * G * D, G * D, qk},
                 {a.QKV + a.nq * D + g * D, D, qk + G * D},
                 {a.QKV + (a.nq + a.nkv) * D + g * D, D, qk + (G + 1) * D}};
    if (!wait_segs<3>(c, sg, tag)) return false;
  }
  stamp(c.a, 1 + 2 * (5 * l + 1));
  // 3. QK-norm (optional) and RoPE: one wave per head, lane j holds the pair (j, j + 64)
  const float* cs = a.rope_cos + (size_t)pos * (D / 2);
  const float* sn = a.rope_sin + (size_t)pos * (D / 2);
  for (int hd = wave; hd < G + 1; hd += kWaves) {
    float* v = qk + hd * D;
    float x0 = v[lane], x1 = v[lane + 64];
    const float* gain = hd < G ? L.q_norm : L.k_norm;
    if (gain) {
      const float ss = wave_sum(x0 * x0 + x1 * x1);
      const float r = 1.0f / sqrtf(ss / (float)D + a.eps);
      x0 = x0 * r * ld_f(gain + lane);
      x1 = x1 * r * ld_f(gain + lane + 64);
    }
    const float ct = ld_f(cs + lane), st = ld_f(sn + lane);
    v[lane] = x0 * ct - x1 * st;
    v[lane + 64] = x1 * ct + x0 * st;
  }
  __syncthreads();
  const float* knew = qk + G * D;
  const float* vnew = qk + (G + 1) * D;
  // 4. the split holding the new position writes its rotated k and raw v to the cache
  if (pos >= p_begin && pos < p_end && threadIdx.x < D) {
    st_f(Kg + (size_t)pos * D + threadIdx.x, knew[threadIdx.x]);
    st_f(Vg + (size_t)pos * D + threadIdx.x, vnew[threadIdx.x]);
  }
  // 5. online softmax over this half-wave's positions
  const float scale = 1.0f / sqrtf((float)D);
  f32x4 qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j) qv[j] = *reinterpret_cast<const f32x4*>(qk + j * D + sub * 4);
  float m[G], ls[G];
  f32x4 o[G];
#pragma unroll
  for (int j = 0; j < G; ++j) { m[j] = -INFINITY; ls[j] = 0.f; o[j] = f32x4{0, 0, 0, 0}; }
  for (int b0 = p_begin + hw; b0 < p_end; b0 += 16 * NP) {
    if (b0 != p_begin + hw) {
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const int p = b0 + 16 * i;
        if (p < p_end && p != pos) {
          kr[i] = ld_f4(Kg + (size_t)p * D + sub * 4);
          vr[i] = ld_f4(Vg + (size_t)p * D + sub * 4);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = b0 + 16 * i;
      if (p < p_end) {
        const f32x4 kv = p == pos ? *reinterpret_cast<const f32x4*>(knew + sub * 4) : kr[i];
        const f32x4 vv = p == pos ? *reinterpret_cast<const f32x4*>(vnew + sub * 4) : vr[i];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float sd = qv[j].x * kv.x + qv[j].y * kv.y + qv[j].z * kv.z + qv[j].w * kv.w;
          sd = group_sum<32>(sd) * scale;
          const float mn = fmaxf(m[j], sd);
          const float corr = __expf(m[j] - mn), pw = __expf(sd - mn);
          ls[j] = ls[j] * corr + pw;
          o[j] = o[j] * corr + vv * pw;
          m[j] = mn;
        }
      }
    }
  }
  // 6. merge the two half-waves of each wave (lanes l and l + 32 hold the same dims)
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const float m2 = __shfl_xor(m[j], 32, 64), l2 = __shfl_xor(ls[j], 32, 64);
    f32x4 o2;
    o2.x = __shfl_xor(o[j].x, 32, 64);
    o2.y = __shfl_xor(o[j].y, 32, 64);
    o2.z = __shfl_xor(o[j].z, 32, 64);
    o2.w = __shfl_xor(o[j].w, 32, 64);
    const float M = fmaxf(m[j], m2);
    if (M != -INFINITY) {
      const float f1 = __expf(m[j] - M), f2 = __expf(m2 - M);
      // lower half first, upper half second: the same order in both halves
      const bool lo = lane < 32;
      const float fa = lo ? f1 : f2, fb = lo ? f2 : f1;
      const float la = lo ? ls[j] : l2, lb = lo ? l2 : ls[j];
      const f32x4 oa = lo ? o[j] : o2, ob = lo ? o2 : o[j];
      ls[j] = la * fa + lb * fb;
      o[j] = oa * fa + ob * fb;
      m[j] = M;
    }
    if (lane < 32) {
      float* e = sm.att + (wave * G + j) * (D + 2);
      *reinterpret_cast<f32x4*>(e + 2 + sub * 4) = o[j];
      if (sub == 0) { e[0] = m[j]; e[1] = ls[j]; }
    }
  }
  __syncthreads();
  // 7. combine the 8 wave states (fixed order) into this split's partial
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D, dd = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.att[(w * G + j) * (D + 2)]);
    float Ls = 0.f, acc = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* e = sm.att + (w * G + j) * (D + 2);
      if (e[0] == -INFINITY) continue;
      const float f = __expf(e[0] - M);
      Ls += e[1] * f;
      acc += e[2 + dd] * f;
    }
    const int h = g * G + j;
    if (S == 1) {
      st_tagged(a.O + h * D + dd, acc / Ls, tag);
    } else {
      uint64_t* dst = a.PART + ((size_t)h * S + s) * (D + 2);
      st_tagged(dst + 2 + dd, acc, tag);
      if (dd == 0) {
        st_tagged(dst, M, tag);
        st_tagged(dst + 1, Ls, tag);
      }
    }
  }
  if (S == 1) {
    stamp(c.a, 2 + 2 * (5 * l + 1));
    return true;
  }
  // 8. heads j with j % S == s are merged here, folding splits 0..S-1 in order
  //    (every split covers at least one position, so l > 0 in each).
  const int nmerge = s < G ? (G - 1 - s) / S + 1 : 0;
  bool ok = true;
  for (int t0 = 0; t0 < nmerge * D; t0 += kThreads) {
    const int t = t0 + threadIdx.x;
    const bool act = t < nmerge * D;
    const int j = s + (t / D) * S, dd = t % D;
    const int h = g * G + j;
    float M = -INFINITY, Ls = 0.f, acc = 0.f;
    for (int q0 = 0; q0 < S && ok; q0 += 8) {
      uint64_t em[8], el[8], eo[8];
      uint32_t spin = 0;
      for (;;) {
        bool done = true;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool in = act && q0 + q < S;
          const uint64_t* e = a.PART + ((size_t)h * S + q0 + q) * (D + 2);
          em[q] = in ? ld_tagged(e) : (uint64_t)tag << 32;
          el[q] = in ? ld_tagged(e + 1) : (uint64_t)tag << 32;
          eo[q] = in ? ld_tagged(e + 2 + dd) : (uint64_t)tag << 32;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          done &= (uint32_t)(em[q] >> 32) == tag && (uint32_t)(el[q] >> 32) == tag && (uint32_t)(eo[q] >> 32) == tag;
        if (done) break;
        if ((++spin & 31) == 0 &&
            (ld_u32(&a.err[0]) != 0 || __builtin_amdgcn_s_memrealtime() - c.t0 > kTimeoutTicks)) {
          st_u32(&a.err[0], 1);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok) break;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (act && q0 + q < S) {
          const float mq = __uint_as_float((uint32_t)em[q]);
          const float lq = __uint_as_float((uint32_t)el[q]);
          const float oq = __uint_as_float((uint32_t)eo[q]);
          const float Mn = fmaxf(M, mq);
          const float fo = __expf(M - Mn), fn = __expf(mq - Mn);
          acc = acc * fo + oq * fn;
          Ls = Ls * fo + lq * fn;
          M = Mn;
        }
      }
    }
    if (ok && act) st_tagged(a.O + h * D + dd, acc / Ls, tag);
  }
  if (!ok) *c.abort_lds = 1;
  __syncthreads();
  stamp(c.a, 2 + 2 * (5 * l + 1));
  return !*c.abort_lds;
}

// Phase C: rows of x1 = x0 + W_o o.  Layer 0 reads x0 = E[token].
__device__ __forceinline__ bool phase_oproj(Ctx& c, Smem& sm, int l, const uint16_t* emb) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  int r0, r1;
  cu_rows(a.H, r0, r1);
  const int K = a.nq * D;
  const SegPlan p = seg_plan(r1 - r0, K);
  const uint16_t* W = L.wo + (size_t)r0 * K;
  auto row = [&](int r) { return W + (size_t)r * K; };
  u32x4 w0[kBatch];
  seg_load(p, p.s0, w0, row);
  zero_part(sm.part, r1 - r0);
  const uint32_t tag = tag_of(c.seq, l);
  float* xres = sm.vec + K;
  if (l == 0) {
    for (int r = threadIdx.x; r < r1 - r0; r += kThreads) xres[r] = bf16_to_f(*gl(emb + r0 + r));
    if (!wait_vec(c, a.O, K, tag, sm.vec)) return false;
  } else {
    Seg sg[2] = {{a.O, K, sm.vec}, {a.X0 + r0, r1 - r0, xres}};
    if (!wait_segs<2>(c, sg, tag)) return false;
  }
  seg_run(p, w0, sm.vec, sm.part, row);
  stamp(c.a, 1 + 2 * (5 * l + 2));
  __syncthreads();
  for (int r = threadIdx.x; r < r1 - r0; r += kThreads) st_tagged(a.X1 + r0 + r, xres[r] + row_total(sm.part, r), tag);
  stamp(c.a, 2 + 2 * (5 * l + 2));
  return true;
}

// Phase D1: act = SiLU(W_g h2) * (W_u h2), h2 = RMSNorm(x1)
__device__ __forceinline__ bool phase_gateup(Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  int i0, i1;
  cu_rows(a.I, i0, i1);
  const int H = a.H;
  const SegPlan p = seg_plan(2 * (i1 - i0), H);  // virtual row 2i = gate row, 2i+1 = up row
  const uint16_t* Wg = L.wg + (size_t)i0 * H;
  const uint16_t* Wu = L.wu + (size_t)i0 * H;
  auto row = [&](int v) { return ((v & 1) ? Wu : Wg) + (size_t)(v >> 1) * H; };
  u32x4 w0[kBatch];
  seg_load(p, p.s0, w0, row);
  zero_part(sm.part, 2 * (i1 - i0));
  const uint32_t tag = tag_of(c.seq, l);
  if (!wait_vec(c, a.X1, H, tag, sm.vec)) return false;
  norm_lds(sm.vec, H, L.mlp_norm, a.eps, sm.red);
  stamp(c.a, 1 + 2 * (5 * l + 3));
  seg_run(p, w0, sm.vec, sm.part, row);
  __syncthreads();
  for (int i = threadIdx.x; i < i1 - i0; i += kThreads) {
    const float gt = row_total(sm.part, 2 * i), up = row_total(sm.part, 2 * i + 1);
    st_tagged(a.ACT + i0 + i, silu_f(gt) * up, tag);
  }
  stamp(c.a, 2 + 2 * (5 * l + 3));
  return true;
}

// Phase D2: rows of x0' = x1 + W_d act
__device__ __forceinline__ bool phase_down(Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  int r0, r1;
  cu_rows(a.H, r0, r1);
  const int K = a.I;
  const SegPlan p = seg_plan(r1 - r0, K);
  const uint16_t* W = L.wd + (size_t)r0 * K;
  auto row = [&](int r) { return W + (size_t)r * K; };
  u32x4 w0[kBatch];
  seg_load(p, p.s0, w0, row);
  zero_part(sm.part, r1 - r0);
  const uint32_t tag = tag_of(c.seq, l);
  float* xres = sm.vec + K;
  Seg sg[2] = {{a.ACT, K, sm.vec}, {a.X1 + r0, r1 - r0, xres}};
  if (!wait_segs<2>(c, sg, tag)) return false;
  seg_run(p, w0, sm.vec, sm.part, row);
  stamp(c.a, 1 + 2 * (5 * l + 4));
  __syncthreads();
  const uint32_t tag_next = tag_of(c.seq, l + 1);
  for (int r = threadIdx.x; r < r1 - r0; r += kThreads) st_tagged(a.X0 + r0 + r, xres[r] + row_total(sm.part, r), tag_next);
  stamp(c.a, 2 + 2 * (5 * l + 4));
  return true;
}

// Final RMSNorm + tied LM head over this CU's vocabulary rows, with the CU's
// argmax (ties -> lowest id) published as a tagged pair.
template <int HS>
__device__ __forceinline__ bool phase_lmhead(Ctx& c, Smem& sm) {
  constexpr int R = 4;  // rows per wave per batch
  const AS4 PersistConst& a = *c.a;
  int v0, v1;
  cu_rows(a.V, v0, v1);
  const int H = a.H, nrows = v1 - v0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint16_t* E = a.embed + (size_t)v0 * H + lane * 8;
  u32x4 wb0[R][HS], wb1[R][HS];
  auto load = [&](u32x4 (&w)[R][HS], int rb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rr = rb + i * kWaves;
      if (rr < nrows) {
#pragma unroll
        for (int sg = 0; sg < HS; ++sg)
          w[i][sg] = ld_w16(E + (size_t)rr * H + sg * kSeg);
      }
    }
  };
  float best = -INFINITY;
  int bi = 0x7fffffff;
  auto consume = [&](const u32x4 (&w)[R][HS], int rb) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int rr = rb + i * kWaves;
      float acc = 0.f;
#pragma unroll
      for (int sg = 0; sg < HS; ++sg) acc += dot8(w[i][sg], sm.vec + sg * kSeg + lane * 8);
      const float t = wave_sum(acc);
      if (rr < nrows) {
        if (lane == 0) st_f(a.logits + v0 + rr, t);
        if (t > best) { best = t; bi = v0 + rr; }  // ids increase within a wave: ties keep the lowest
      }
    }
  };
  load(wb0, wave);
  if (!wait_vec(c, a.X0, H, tag_of(c.seq, a.L), sm.vec)) return false;
  norm_lds(sm.vec, H, a.final_norm, a.eps, sm.red);
  stamp(c.a, 1 + 2 * (5 * a.L));
  if (blockIdx.x == 0 && a.xf_out)
    for (int k = threadIdx.x; k < H; k += kThreads) st_f(a.xf_out + k, sm.vec[k]);
  constexpr int step = R * kWaves;
  for (int rb = wave; rb < nrows; rb += 2 * step) {
    if (rb + step < nrows) load(wb1, rb + step);
    consume(wb0, rb);
    if (rb + 2 * step < nrows) load(wb0, rb + 2 * step);
    if (rb + step < nrows) consume(wb1, rb + step);
  }
  float* bv = sm.red;
  int* bj = reinterpret_cast<int*>(sm.red + kWaves);
  if (lane == 0) { bv[wave] = best; bj[wave] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = bv[0];
    int j = bj[0];
    for (int w = 1; w < kWaves; ++w)
      if (bv[w] > v || (bv[w] == v && bj[w] < j)) { v = bv[w]; j = bj[w]; }
    st_tagged(a.AMV + blockIdx.x, v, tag_of(c.seq, 255));
    st_tagged(a.AMI + blockIdx.x, __int_as_float(j), tag_of(c.seq, 255));
  }
  stamp(c.a, 2 + 2 * (5 * a.L));
  return true;
}

// CU 0: argmax over the per-CU partials (ties -> lowest id); advance the step state.
__device__ __forceinline__ void phase_final(Ctx& c, Smem& sm) {
  const AS4 PersistConst& a = *c.a;
  if (blockIdx.x != 0) return;
  const int n = gridDim.x;
  float* vals = sm.vec;
  float* idxs = sm.vec + n;
  Seg sg[2] = {{a.AMV, n, vals}, {a.AMI, n, idxs}};
  if (!wait_segs<2>(c, sg, tag_of(c.seq, 255))) return;
  stamp(c.a, 1 + 2 * (5 * a.L + 1));
  if (threadIdx.x < 64) {
    // (value desc, id asc) is a total order, so the result does not depend on the scan order
    float v = -INFINITY;
    int j = 0x7fffffff;
    for (int i = threadIdx.x; i < n; i += 64) {
      const float vi = vals[i];
      const int ji = __float_as_int(idxs[i]);
      if (vi > v || (vi == v && ji < j)) { v = vi; j = ji; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(v, off, 64);
      const int oj = __shfl_xor(j, off, 64);
      if (ov > v || (ov == v && oj < j)) { v = ov; j = oj; }
    }
    if (threadIdx.x == 0) {
      if (j == 0x7fffffff) j = 0;  // only if every logit was NaN
      AS1 DevState* st = gl(a.st);
      st->token = j;
      st->pos = c.pos + 1;
      st->step += 1;
    }
  }
  stamp(c.a, 2 + 2 * (5 * a.L + 1));
}

template <int G, int HS>
__global__ __launch_bounds__(kThreads, 1) void k_decode_persistent(const PersistConst* __restrict__ pc, int pos,
                                                                   uint32_t seq, int S, int chunk) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  if (threadIdx.x == 0) sm.abort_flag = 0;
  __syncthreads();
  const AS4 PersistConst* a = (const AS4 PersistConst*)pc;
  Ctx c{a, pos, S, chunk, seq, __builtin_amdgcn_s_memrealtime(), &sm.abort_flag};
  stamp(a, 0);
  const uint16_t* emb = a->embed + (size_t)gl(a->st)->token * a->H;
  const int L = a->L;
  for (int l = 0; l < L; ++l) {
    if (!phase_qkv(c, sm, l, emb)) return;
    if (!phase_attn<G>(c, sm, l)) return;
    if (!phase_oproj(c, sm, l, emb)) return;
    if (!phase_gateup(c, sm, l)) return;
    if (!phase_down(c, sm, l)) return;
  }
  if (!phase_lmhead<HS>(c, sm)) return;
  phase_final(c, sm);
}

template <int G, int HS>
void* kernel_ptr() {
  return (void*)k_decode_persistent<G, HS>;
}

void* pick(int G, int hseg) {
  if (hseg == 2) {
    switch (G) {
      case 1: return kernel_ptr<1, 2>();
      case 2: return kernel_ptr<2, 2>();
      case 4: return kernel_ptr<4, 2>();
      case 8: return kernel_ptr<8, 2>();
    }
  } else if (hseg == 4) {
    switch (G) {
      case 1: return kernel_ptr<1, 4>();
      case 2: return kernel_ptr<2, 4>();
      case 4: return kernel_ptr<4, 4>();
      case 8: return kernel_ptr<8, 4>();
    }
  }
  return nullptr;
}

}  // namespace

size_t persist_smem_bytes() { return sizeof(Smem); }

int persist_prepare(int G, int hseg) {
  void* fn = pick(G, hseg);
  if (!fn) return -1;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
  return e == hipSuccess ? 0 : (int)e;
}

int persist_launch(const PersistConst* dev_const, int G, int hseg, int grid, int pos, uint32_t seq, int S, int chunk,
                   hipStream_t s) {
  void* fn = pick(G, hseg);
  if (!fn) return -1;
  void* args[] = {(void*)&dev_const, (void*)&pos, (void*)&seq, (void*)&S, (void*)&chunk};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kThreads), args, sizeof(Smem), s);
  return e == hipSuccess ? 0 : (int)e;
}
