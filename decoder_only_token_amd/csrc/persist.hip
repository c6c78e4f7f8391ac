// Persistent decode step for gfx950: the whole single-token forward in ONE
// cooperative kernel launch, one 512-thread workgroup (8 waves) per CU.
//
// A decode step is a chain of ~5 dependent phases per layer.  As separate
// kernels every dependency costs a launch gap plus the ramp and tail of the
// next kernel; here each dependency is a device-scope handshake instead.
// Producers publish every value as a 64-bit word {f32 value | tag << 32} with
// one relaxed agent-scope store; consumers spin with relaxed agent-scope loads
// until every word carries the tag they expect.  No fences, no shared
// counters, no L2 writeback/invalidate: the tag itself says the value is there.
//
// Phases of layer l (tag = seq << 8 | l unless noted):
//   A  rows of q|k|v = W_qkv RMSNorm(x0) + b                       -> QKV
//   B  attention item (kv head g, split s): QK-norm, RoPE, KV-cache write,
//      online softmax over its positions; split partials merged     -> O
//   C  rows of x1 = x0 + W_o o                                       -> X1
//   D1 rows of act = SiLU(W_g h2) * (W_u h2), h2 = RMSNorm(x1)        -> ACT
//   D2 rows of x0' = x1 + W_d act                                    -> X0 (tag l+1)
// then the final RMSNorm + tied LM head with per-CU argmax partials, and the
// argmax over the partials by CU 0, which advances the step state.
//
// Every phase: all 512 threads poll the input (a few values each) into LDS,
// one workgroup barrier, then each wave computes whole output rows from
// weights that were loaded into registers at the end of the PREVIOUS phase, so
// the weight stream overlaps the handshake.  RMSNorm is folded in: the LDS
// input is gain * x and each row sum is scaled by 1/RMS(x) afterwards.
//
// The fused QKV rows are stored group-major ([kv head g][q heads of g | k_g |
// v_g] x 128), so one attention item reads one contiguous run.
//
// Reusing a buffer across phases is safe: every reader of a buffer instance
// is, through the dataflow, a required producer of what the next writer of
// that buffer waits for.  This needs every CU to own at least one row of the
// QKV, hidden and intermediate projections (the host checks it), and every
// LDS input slot is rewritten only after a workgroup barrier that all waves
// reach after their last read of it.
#include "common.h"
#include "persist.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kSeg = 512;  // bf16 per segment: 64 lanes x 8 values (16 bytes)
constexpr int kBatch = 8;  // segments per wave per load batch
constexpr int D = 128;     // head_dim
constexpr int kVecMax = 11264;
constexpr int kAttStride = D + 4;  // {m, l, -, -, o[128]}: o stays 16-byte aligned
constexpr int kPE = 8;             // tagged values per thread per poll pass (4096 per pass)
constexpr uint64_t kTimeoutTicks = 20000000ull;  // 200 ms of the 100 MHz real-time counter

// Explicit address spaces: pointers read from the parameter block would stay
// generic, and FLAT instructions also count against the LDS wait counter.
// AS1 = global memory, AS4 = constant (uniform data, scalar loads).
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
__device__ __forceinline__ float ld_f(const float* p) { return *gl(p); }
__device__ __forceinline__ void st_f(float* p, float v) { *gl(p) = v; }
__device__ __forceinline__ uint32_t tag_of(uint32_t seq, int l) { return (seq << 8) | (uint32_t)l; }

__device__ __forceinline__ f32x4 as_f4(u32x4 u) {
  return f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}

// Cross-lane sums with DPP in a fixed order.
#define DPPF(v, ctrl, rmask) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, false))
__device__ __forceinline__ float row16_sum(float v) {  // every lane: the sum of its row of 16 lanes
  v += DPPF(v, 0xB1, 0xF);   // quad_perm [1,0,3,2]
  v += DPPF(v, 0x4E, 0xF);   // quad_perm [2,3,0,1]
  v += DPPF(v, 0x141, 0xF);  // row_half_mirror
  v += DPPF(v, 0x140, 0xF);  // row_mirror
  return v;
}
__device__ __forceinline__ float wave_total(float v) {  // the sum of all 64 lanes, in every lane
  v = row16_sum(v);
  v += DPPF(v, 0x142, 0xA);  // row_bcast:15 -> rows 1, 3
  v += DPPF(v, 0x143, 0xC);  // row_bcast:31 -> rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float half_total(float v) {  // the sum of this lane's half-wave (32 lanes)
  v = row16_sum(v);
  v += DPPF(v, 0x142, 0xA);
  const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
  const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  return (threadIdx.x & 32) ? hi : lo;
}

struct Smem {
  float vec[2][kVecMax];  // phase inputs (gain * x for normed phases), slot = phase & 1
  float xres[2][64];      // residual rows of this CU, slot = phase & 1
  float att[kWaves * 8 * kAttStride];
  float qk[10 * D];  // rotated q heads, k, v of one kv group
  float red[48];     // [0, 16): RMS partials by phase parity; [32, 48): LM-head argmax
  int abort_flag;
};

struct Ctx {
  const AS4 PersistConst* a;
  int pos, S, chunk;
  uint32_t seq;
  uint64_t t0;
  // this CU's row ranges, computed once: fused qkv rows, hidden rows,
  // intermediate rows, vocabulary rows
  int q0, q1, h0, h1, i0, i1, v0, v1;
};

// rows [r0, r1) of N split evenly over the grid (32-bit: N * grid < 2^31)
__device__ __forceinline__ void cu_rows(int N, int& r0, int& r1) {
  r0 = (int)(((uint32_t)N * blockIdx.x) / gridDim.x);
  r1 = (int)(((uint32_t)N * (blockIdx.x + 1)) / gridDim.x);
}

__device__ __forceinline__ void stamp(const Ctx& c, int ph, int what, bool who) {
  if (c.a->trace && who)
    *gl(c.a->trace + (size_t)blockIdx.x * persist_trace_slots(c.a->L) + ph * kTraceSlots + what) =
        __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ bool timed_out(const Ctx& c) {
  return ld_u32(&c.a->err[0]) != 0 || __builtin_amdgcn_s_memrealtime() - c.t0 > kTimeoutTicks;
}

// ------------------------------------------------------------------ polling
// All 512 threads: copy n tagged values src[0..n) (and n2 <= 64 values
// src2[0..n2) to dst2) into LDS once every tag equals `tag`.  With `gain`, the
// LDS copy is gain[k] * x[k] and *rs receives 1 / sqrt(mean(x^2) + eps), the
// RMSNorm scale, applied to the row sums later.  Ends with a workgroup
// barrier; returns false on every thread when the step is abandoned.
__device__ bool poll(const Ctx& c, Smem& sm, int ph, const uint64_t* src, int n, uint32_t tag, float* dst,
                     const float* gain, float* rs, const uint64_t* src2, int n2, float* dst2) {
  const int tid = threadIdx.x;
  bool ok = !sm.abort_flag;
  float ss = 0.f;
  for (int base = 0; ok && base < n; base += kPE * kThreads) {
    float gv[kPE];
    if (gain) {
#pragma unroll
      for (int e = 0; e < kPE; ++e) {
        const int i = base + e * kThreads + tid;
        gv[e] = i < n ? ld_f(gain + i) : 0.f;
      }
    }
    const uint64_t want = (uint64_t)tag << 32;
    uint64_t v[kPE], v2 = want;
    uint32_t spin = 0;
    for (;;) {
      bool done = true;
#pragma unroll
      for (int e = 0; e < kPE; ++e) {
        const int i = base + e * kThreads + tid;
        v[e] = i < n ? ld_tagged(src + i) : want;
      }
      if (base == 0 && tid < n2) v2 = ld_tagged(src2 + tid);
#pragma unroll
      for (int e = 0; e < kPE; ++e) done &= (uint32_t)(v[e] >> 32) == tag;
      done &= (uint32_t)(v2 >> 32) == tag;
      if (done) break;
      if ((++spin & 31) == 0 && timed_out(c)) {
        st_u32(&c.a->err[0], 1);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) break;
#pragma unroll
    for (int e = 0; e < kPE; ++e) {
      const int i = base + e * kThreads + tid;
      if (i < n) {
        const float x = __uint_as_float((uint32_t)v[e]);
        dst[i] = gain ? x * gv[e] : x;
        ss += x * x;
      }
    }
    if (base == 0 && tid < n2) dst2[tid] = __uint_as_float((uint32_t)v2);
  }
  if (!ok) sm.abort_flag = 1;
  float* red = sm.red + (ph & 1) * 8;
  if (gain) {
    const float w = wave_total(ss);
    if ((tid & 63) == 0) red[tid >> 6] = w;
  }
  __syncthreads();
  if (sm.abort_flag) return false;
  if (gain) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += red[i];
    *rs = rsqrtf(t / (float)n + c.a->eps);
  }
  return true;
}

// ------------------------------------------------------------ phase geometry
enum { kQKV = 0, kAttn = 1, kOproj = 2, kGateUp = 3, kDown = 4 };

// A GEMV phase: units (one row, or a gate/up row pair) [0, nunits) of this
// CU; unit u belongs to wave u % 8 and covers `rpu` rows of K values, read in
// segments of 512.
struct Gemv {
  const uint16_t* a;  // first row of this CU's slice (gate rows for pairs)
  long delta;         // up rows - gate rows, in elements (pairs only)
  int K, nseg, rpu, nunits, r0;
};

__device__ __forceinline__ Gemv gemv_of(const Ctx& c, int l, int kind) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  Gemv g;
  g.delta = 0;
  g.rpu = 1;
  switch (kind) {
    case kQKV: g.r0 = c.q0; g.nunits = c.q1 - c.q0; g.K = a.H; g.a = L.wqkv; break;
    case kOproj: g.r0 = c.h0; g.nunits = c.h1 - c.h0; g.K = a.nq * D; g.a = L.wo; break;
    case kGateUp:
      g.r0 = c.i0; g.nunits = c.i1 - c.i0; g.K = a.H; g.a = L.wg; g.delta = (long)(L.wu - L.wg); g.rpu = 2;
      break;
    default: g.r0 = c.h0; g.nunits = c.h1 - c.h0; g.K = a.I; g.a = L.wd; break;
  }
  g.a += (size_t)g.r0 * g.K;
  g.nseg = (g.K + kSeg - 1) / kSeg;
  return g;
}

// A wave's walk over its segments: unit u (= wave + 8 j), row-in-unit t, segment sg.
struct Walk {
  int u, t, sg;
};

__device__ __forceinline__ bool walk_valid(const Gemv& g, const Walk& w) { return w.u < g.nunits; }

__device__ __forceinline__ void walk_next(const Gemv& g, Walk& w) {
  if (++w.sg == g.nseg) {
    w.sg = 0;
    if (++w.t == g.rpu) {
      w.t = 0;
      w.u += kWaves;
    }
  }
}

// Always inside this CU's rows (nunits >= 1): a wave without units, and the
// tail of a row shorter than a whole segment, re-read valid data.
__device__ __forceinline__ const uint16_t* seg_ptr(const Gemv& g, const Walk& w) {
  const int lane = threadIdx.x & 63;
  const int k = min(w.sg * kSeg + lane * 8, g.K - 8);
  return g.a + (long)w.t * g.delta + (long)min(w.u, g.nunits - 1) * g.K + k;
}

// ----------------------------------------------------------------- registers
// The phase's first batch (weight segments, or the K/V rows of the attention
// item: K in R[0..3], V in R[4..7]) is loaded at ONE program point of the
// phase loop; each phase only computes addresses.  Values defined on several
// paths would be merged with register copies, and a copy waits for its load.
struct Regs {
  u32x4 R[kBatch];
};
struct Addr {
  const u32x4* p[kBatch];
};

__device__ __forceinline__ void load_regs(Regs& rg, const Addr& ad) {
#pragma unroll
  for (int i = 0; i < kBatch; ++i) rg.R[i] = __builtin_nontemporal_load(gl(ad.p[i]));
}

// Addresses of the next 8 segments from walk position w (the last valid
// segment repeats past the end, so every register is loaded).
__device__ __forceinline__ void gemv_addr(Addr& ad, const Gemv& g, Walk w) {
  Walk last = w;
#pragma unroll
  for (int i = 0; i < kBatch; ++i) {
    if (walk_valid(g, w)) last = w;
    ad.p[i] = reinterpret_cast<const u32x4*>(seg_ptr(g, last));
    walk_next(g, w);
  }
}

// Attention batch b: positions p_begin + hw + 16 (b + i), i < 4, for the 16
// half-waves hw (clamped into the split).
__device__ __forceinline__ void kv_addr(Addr& ad, const float* Kg, const float* Vg, int p_begin, int p_end, int b) {
  const int hw = threadIdx.x >> 5, sub = threadIdx.x & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = min(p_begin + hw + 16 * (b + i), p_end - 1);
    ad.p[i] = reinterpret_cast<const u32x4*>(Kg + (size_t)p * D + sub * 4);
    ad.p[4 + i] = reinterpret_cast<const u32x4*>(Vg + (size_t)p * D + sub * 4);
  }
}

// LM head: rows rb, rb + 8, ... (kBatch / HS rows of HS segments) of this
// CU's vocabulary slice, clamped into it.
template <int HS>
__device__ __forceinline__ void lm_addr(Addr& ad, const uint16_t* E, int rb, int nrows) {
#pragma unroll
  for (int i = 0; i < kBatch / HS; ++i) {
    const int rr = min(rb + i * kWaves, nrows - 1);
#pragma unroll
    for (int sg = 0; sg < HS; ++sg)
      ad.p[i * HS + sg] = reinterpret_cast<const u32x4*>(E + (size_t)rr * HS * kSeg + sg * kSeg);
  }
}

__device__ __forceinline__ bool has_item(const Ctx& c) { return (int)blockIdx.x < c.a->nkv * c.S; }

// First-batch addresses of phase ph (ph == 5 L: the LM head).
template <int HS>
__device__ __forceinline__ Addr phase_addr(const Ctx& c, int ph) {
  const AS4 PersistConst& a = *c.a;
  const int l = ph / 5, kind = ph % 5, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  Addr ad;
  if (l >= a.L) {
    lm_addr<HS>(ad, a.embed + (size_t)c.v0 * HS * kSeg + lane * 8, wave, c.v1 - c.v0);
  } else if (kind == kAttn) {
    if (!has_item(c)) {  // no item: same-address loads keep the registers defined
#pragma unroll
      for (int i = 0; i < kBatch; ++i) ad.p[i] = reinterpret_cast<const u32x4*>(a.Kc);
    } else {
      const int g = blockIdx.x / c.S, s = blockIdx.x % c.S;
      const int p_begin = s * c.chunk, p_end = min(p_begin + c.chunk, c.pos + 1);
      kv_addr(ad, a.Kc + ((size_t)l * a.nkv + g) * a.max_pos * D, a.Vc + ((size_t)l * a.nkv + g) * a.max_pos * D,
              p_begin, p_end, 0);
    }
  } else {
    const Gemv g = gemv_of(c, l, kind);
    gemv_addr(ad, g, Walk{wave, 0, 0});
  }
  return ad;
}

// ------------------------------------------------------------------- phases
// GEMV phase: this wave's units, the first batch from rg and further batches
// through a local array; each finished row goes straight to its output word.
__device__ __forceinline__ void gemv_phase(const Ctx& c, Smem& sm, int l, int kind, const Regs& rg, float rs) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const int ph = 5 * l + kind, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const Gemv g = gemv_of(c, l, kind);
  const float* h = sm.vec[ph & 1];
  const float* xr = sm.xres[ph & 1];
  const uint32_t tag = tag_of(c.seq, l);
  Walk w{wave, 0, 0};
  float acc = 0.f, first = 0.f;
  auto consume = [&](const Regs& r) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (walk_valid(g, w)) {  // wave-uniform
        const int k = w.sg * kSeg + lane * 8;
        if (k < g.K) acc += dot8(r.R[i], h + k);
        if (w.sg + 1 == g.nseg) {  // row finished
          const float t = wave_total(acc) * rs;
          acc = 0.f;
          if (w.t + 1 < g.rpu) {
            first = t;  // gate row of a pair
          } else if (lane == 0) {
            const int r = g.r0 + w.u;
            switch (kind) {
              case kQKV: st_tagged(a.QKV + r, Lw.bqkv ? t + ld_f(Lw.bqkv + r) : t, tag); break;
              case kOproj: st_tagged(a.X1 + r, xr[w.u] + t, tag); break;
              case kGateUp: st_tagged(a.ACT + r, silu_f(first) * t, tag); break;
              default: st_tagged(a.X0 + r, xr[w.u] + t, tag_of(c.seq, l + 1)); break;
            }
          }
        }
        walk_next(g, w);
      }
    }
  };
  consume(rg);
  while (walk_valid(g, w)) {  // more than one batch
    Addr ad;
    gemv_addr(ad, g, w);
    Regs r2;
    load_regs(r2, ad);
    consume(r2);
  }
}

// Attention item (kv head g, split s), part 1: QK-norm + RoPE of the q heads
// and k in LDS, the new cache row, then online softmax over positions
// p_begin + hw + 16 i (hw = the 16 half-waves; a lane holds 4 of the 128
// dims), the two half-waves merged, per-wave state into LDS.
template <int G>
__device__ __forceinline__ void attn_phase(const Ctx& c, Smem& sm, int l, const Regs& rg) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const int S = c.S, pos = c.pos, ctx = pos + 1;
  const int g = blockIdx.x / S, s = blockIdx.x % S;
  const int p_begin = s * c.chunk, p_end = min(p_begin + c.chunk, ctx);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, hw = threadIdx.x >> 5, sub = lane & 31;
  float* Kg = a.Kc + ((size_t)l * a.nkv + g) * a.max_pos * D;
  float* Vg = a.Vc + ((size_t)l * a.nkv + g) * a.max_pos * D;
  float* qk = sm.qk;
  // QK-norm (optional) and RoPE; wave hd handles head hd (lane j: the pair (j, j + 64))
  for (int hd = wave; hd < G + 1; hd += kWaves) {
    float* v = qk + hd * D;
    float x0 = v[lane], x1 = v[lane + 64];
    const float* gain = hd < G ? Lw.q_norm : Lw.k_norm;
    if (gain) {
      const float r = rsqrtf(wave_total(x0 * x0 + x1 * x1) / (float)D + a.eps);
      x0 = x0 * r * ld_f(gain + lane);
      x1 = x1 * r * ld_f(gain + lane + 64);
    }
    const float ct = ld_f(a.rope_cos + (size_t)pos * (D / 2) + lane);
    const float st = ld_f(a.rope_sin + (size_t)pos * (D / 2) + lane);
    v[lane] = x0 * ct - x1 * st;
    v[lane + 64] = x1 * ct + x0 * st;
  }
  __syncthreads();
  const float* knew = qk + G * D;
  const float* vnew = qk + (G + 1) * D;
  if (pos >= p_begin && pos < p_end && threadIdx.x < D) {  // this split holds the new position
    st_f(Kg + (size_t)pos * D + threadIdx.x, knew[threadIdx.x]);
    st_f(Vg + (size_t)pos * D + threadIdx.x, vnew[threadIdx.x]);
  }
  const float scale = 1.0f / sqrtf((float)D);
  f32x4 qv[G];
#pragma unroll
  for (int j = 0; j < G; ++j) qv[j] = *reinterpret_cast<const f32x4*>(qk + j * D + sub * 4);
  float m[G], ls[G];
  f32x4 o[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    ls[j] = 0.f;
    o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int wave_first = p_begin + 2 * wave;  // this wave's lower-half position in batch 0
  auto consume = [&](const Regs& r, int b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (wave_first + 16 * (b + i) < p_end) {  // wave-uniform: the lower half has a position
        const int p = p_begin + hw + 16 * (b + i);
        const bool valid = p < p_end;
        // the cache row of the new position was prefetched before it was written
        const f32x4 kv = p == pos ? *reinterpret_cast<const f32x4*>(knew + sub * 4) : as_f4(r.R[i]);
        const f32x4 vv = p == pos ? *reinterpret_cast<const f32x4*>(vnew + sub * 4) : as_f4(r.R[4 + i]);
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float sd = qv[j].x * kv.x + qv[j].y * kv.y + qv[j].z * kv.z + qv[j].w * kv.w;
          sd = half_total(sd) * scale;
          if (valid) {
            const float mn = fmaxf(m[j], sd);
            const float corr = __expf(m[j] - mn), pw = __expf(sd - mn);
            ls[j] = ls[j] * corr + pw;
            o[j] = o[j] * corr + vv * pw;
            m[j] = mn;
          }
        }
      }
    }
  };
  consume(rg, 0);
  for (int b = 4; wave_first + b * 16 < p_end; b += 4) {
    Addr ad;
    kv_addr(ad, Kg, Vg, p_begin, p_end, b);
    Regs r2;
    load_regs(r2, ad);
    consume(r2, b);
  }
  // merge the two half-waves of this wave, lower half first (same order in both halves)
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
      const bool lo = lane < 32;
      const float fa = __expf((lo ? m[j] : m2) - M), fb = __expf((lo ? m2 : m[j]) - M);
      const float la = lo ? ls[j] : l2, lb = lo ? l2 : ls[j];
      const f32x4 oa = lo ? o[j] : o2, ob = lo ? o2 : o[j];
      ls[j] = la * fa + lb * fb;
      o[j] = oa * fa + ob * fb;
      m[j] = M;
    }
    if (lane < 32) {
      float* e = sm.att + (wave * G + j) * kAttStride;
      *reinterpret_cast<f32x4*>(e + 4 + sub * 4) = o[j];
      if (sub == 0) {
        e[0] = m[j];
        e[1] = ls[j];
      }
    }
  }
}

// Attention item, part 2: combine the 8 wave states in a fixed order into this
// split's partial (with one split, into the output); then the heads j with
// j % S == s fold the S split partials in split order.
template <int G>
__device__ __forceinline__ bool attn_finish(const Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const int S = c.S, g = blockIdx.x / S, s = blockIdx.x % S;
  const uint32_t tag = tag_of(c.seq, l);
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int j = idx / D, dd = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.att[(w * G + j) * kAttStride]);
    float Ls = 0.f, acc = 0.f;
    for (int w = 0; w < kWaves; ++w) {
      const float* e = sm.att + (w * G + j) * kAttStride;
      if (e[0] == -INFINITY) continue;  // a wave without positions
      const float f = __expf(e[0] - M);
      Ls += e[1] * f;
      acc += e[4 + dd] * f;
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
  if (S == 1) return true;
  const int nmerge = s < G ? (G - 1 - s) / S + 1 : 0;
  bool ok = true;
  for (int t0 = 0; t0 < nmerge * D; t0 += kThreads) {
    const int t = t0 + threadIdx.x;
    const bool act = t < nmerge * D;
    const int j = s + (t / D) * S, dd = t % D;
    const int h = g * G + (act ? j : 0);
    float M = -INFINITY, Ls = 0.f, acc = 0.f;
    for (int q0 = 0; q0 < S && ok; q0 += 8) {
      uint64_t em[8], el[8], eo[8];
      uint32_t spin = 0;
      const uint64_t dflt = (uint64_t)tag << 32;
      for (;;) {
        bool done = true;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const bool in = act && q0 + q < S;
          const uint64_t* e = a.PART + ((size_t)h * S + min(q0 + q, S - 1)) * (D + 2);
          em[q] = in ? ld_tagged(e) : dflt;
          el[q] = in ? ld_tagged(e + 1) : dflt;
          eo[q] = in ? ld_tagged(e + 2 + dd) : dflt;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          done &= (uint32_t)(em[q] >> 32) == tag && (uint32_t)(el[q] >> 32) == tag && (uint32_t)(eo[q] >> 32) == tag;
        if (done) break;
        if ((++spin & 31) == 0 && timed_out(c)) {
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
          const float mq = __uint_as_float((uint32_t)em[q]), lq = __uint_as_float((uint32_t)el[q]);
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
  if (!ok) sm.abort_flag = 1;
  __syncthreads();
  return !sm.abort_flag;
}

// LM head: rows wave, wave + 8, ... of this CU's vocabulary slice (first batch
// in rg), logits out, per-CU argmax (ties -> lowest id) as a tagged pair.
template <int HS>
__device__ __forceinline__ void lmhead_phase(const Ctx& c, Smem& sm, Regs& rg, float rs) {
  const AS4 PersistConst& a = *c.a;
  constexpr int RB = kBatch / HS;  // rows per batch
  const int v0 = c.v0, nrows = c.v1 - c.v0, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* h = sm.vec[(5 * a.L) & 1];
  const uint16_t* E = a.embed + (size_t)v0 * HS * kSeg + lane * 8;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  auto consume = [&](const Regs& src, int rb) {
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rr = rb + i * kWaves;
      if (rr < nrows) {  // wave-uniform
        float acc = 0.f;
#pragma unroll
        for (int sg = 0; sg < HS; ++sg) acc += dot8(src.R[i * HS + sg], h + sg * kSeg + lane * 8);
        const float t = wave_total(acc) * rs;
        if (lane == 0) st_f(a.logits + v0 + rr, t);
        if (t > best) {  // a wave's rows increase: ties keep the lowest id
          best = t;
          bi = v0 + rr;
        }
      }
    }
  };
  constexpr int step = RB * kWaves;
  Regs r2;
  Addr ad;
  for (int rb = wave; rb < nrows; rb += 2 * step) {
    lm_addr<HS>(ad, E, rb + step, nrows);
    load_regs(r2, ad);
    consume(rg, rb);
    lm_addr<HS>(ad, E, rb + 2 * step, nrows);
    load_regs(rg, ad);
    consume(r2, rb + step);
  }
  if (lane == 0) {
    sm.red[32 + wave] = best;
    sm.red[40 + wave] = __int_as_float(bi);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = sm.red[32];
    int j = __float_as_int(sm.red[40]);
    for (int w = 1; w < kWaves; ++w) {
      const float vw = sm.red[32 + w];
      const int jw = __float_as_int(sm.red[40 + w]);
      if (vw > v || (vw == v && jw < j)) {
        v = vw;
        j = jw;
      }
    }
    st_tagged(a.AM + 2 * blockIdx.x, v, tag_of(c.seq, 255));
    st_tagged(a.AM + 2 * blockIdx.x + 1, __int_as_float(j), tag_of(c.seq, 255));
  }
}

// CU 0: argmax over the per-CU {value, id} pairs; (value desc, id asc) is a
// total order, so the scan order does not matter.  Advances the step state.
__device__ __forceinline__ void final_phase(const Ctx& c, Smem& sm) {
  const AS4 PersistConst& a = *c.a;
  const int n = gridDim.x, ph = 5 * a.L + 1;
  float* vals = sm.vec[ph & 1];
  float rs;
  stamp(c, ph, 0, threadIdx.x == 0);
  if (!poll(c, sm, ph, a.AM, 2 * n, tag_of(c.seq, 255), vals, nullptr, &rs, nullptr, 0, nullptr)) return;
  stamp(c, ph, 1, threadIdx.x == 0);
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float v = -INFINITY;
  int j = 0x7fffffff;
  for (int i = lane; i < n; i += 64) {
    const float vi = vals[2 * i];
    const int ji = __float_as_int(vals[2 * i + 1]);
    if (vi > v || (vi == v && ji < j)) {
      v = vi;
      j = ji;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off, 64);
    const int oj = __shfl_xor(j, off, 64);
    if (ov > v || (ov == v && oj < j)) {
      v = ov;
      j = oj;
    }
  }
  if (lane == 0) {
    if (j == 0x7fffffff) j = 0;  // only if every logit was NaN
    AS1 DevState* st = gl(a.st);
    st->token = j;
    st->pos = c.pos + 1;
    st->step += 1;
  }
  stamp(c, ph, 5, lane == 0);
}

template <int G, int HS>
__global__ __launch_bounds__(kThreads, 1) void k_decode_persistent(const PersistConst* __restrict__ pc, int pos,
                                                                   uint32_t seq, int S, int chunk) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  if (threadIdx.x == 0) sm.abort_flag = 0;
  const AS4 PersistConst* ap = (const AS4 PersistConst*)pc;
  const AS4 PersistConst& a = *ap;
  Ctx c{ap, pos, S, chunk, seq, __builtin_amdgcn_s_memrealtime()};
  cu_rows(a.nqkv, c.q0, c.q1);
  cu_rows(a.H, c.h0, c.h1);
  cu_rows(a.I, c.i0, c.i1);
  cu_rows(a.V, c.v0, c.v1);
  stamp(c, 0, 7, threadIdx.x == 0);
  const int L = a.L, H = a.H, tid = threadIdx.x;
  const uint16_t* emb = a.embed + (size_t)gl(a.st)->token * H;
  Regs rg;
  load_regs(rg, phase_addr<HS>(c, 0));
  __syncthreads();
  for (int ph = 0; ph < 5 * L; ++ph) {
    const int l = ph / 5, kind = ph % 5;
    const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
    const uint32_t tag = tag_of(seq, l);
    float* vin = sm.vec[ph & 1];
    float* xr = sm.xres[ph & 1];
    float rs = 1.0f;
    const bool item = kind != kAttn || has_item(c);
    stamp(c, ph, 0, tid == 0);
    // ---- the phase input
    bool ok = true;
    if (!item) {
      __syncthreads();  // keeps the workgroup barrier sequence of the other CUs
    } else if (l == 0 && kind == kQKV) {  // layer 0: x0 is the embedding row (nothing to wait for)
      float ss = 0.f;
      for (int k = tid; k < H; k += kThreads) {
        const float x = bf16_to_f(*gl(emb + k));
        vin[k] = x * ld_f(Lw.attn_norm + k);
        ss += x * x;
      }
      const float wsum = wave_total(ss);
      if ((tid & 63) == 0) sm.red[tid >> 6] = wsum;
      __syncthreads();
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) t += sm.red[i];
      rs = rsqrtf(t / (float)H + a.eps);
    } else {
      const uint64_t* src;
      const uint64_t* src2 = nullptr;
      const float* gain = nullptr;
      int n, n2 = 0;
      float* dst = vin;
      switch (kind) {
        case kQKV: src = a.X0; n = H; gain = Lw.attn_norm; break;
        case kAttn: src = a.QKV + (size_t)(blockIdx.x / S) * (G + 2) * D; n = (G + 2) * D; dst = sm.qk; break;
        case kOproj:
          src = a.O;
          n = a.nq * D;
          if (l == 0) {
            for (int r = tid; r < c.h1 - c.h0; r += kThreads) xr[r] = bf16_to_f(*gl(emb + c.h0 + r));
          } else {
            src2 = a.X0 + c.h0;
            n2 = c.h1 - c.h0;
          }
          break;
        case kGateUp: src = a.X1; n = H; gain = Lw.mlp_norm; break;
        default: src = a.ACT; n = a.I; src2 = a.X1 + c.h0; n2 = c.h1 - c.h0; break;
      }
      ok = poll(c, sm, ph, src, n, tag, dst, gain, &rs, src2, n2, xr);
    }
    if (!ok) return;
    stamp(c, ph, 1, tid == 0);
    // ---- compute from the registers loaded at the end of the previous phase
    if (kind == kAttn) {
      if (item) attn_phase<G>(c, sm, l, rg);
    } else {
      gemv_phase(c, sm, l, kind, rg, rs);
    }
    stamp(c, ph, 3, tid == 0);
    // the single load site: the next phase's first batch flies during the handshake
    load_regs(rg, phase_addr<HS>(c, ph + 1));
    if (kind == kAttn && item && !attn_finish<G>(c, sm, l)) return;
    stamp(c, ph, 5, tid == 0);
  }
  // ---- final norm + LM head
  {
    const int ph = 5 * L;
    float rs;
    stamp(c, ph, 0, tid == 0);
    if (!poll(c, sm, ph, a.X0, H, tag_of(seq, L), sm.vec[ph & 1], a.final_norm, &rs, nullptr, 0, nullptr)) return;
    stamp(c, ph, 1, tid == 0);
    if (blockIdx.x == 0 && a.xf_out)
      for (int k = tid; k < H; k += kThreads) st_f(a.xf_out + k, sm.vec[ph & 1][k] * rs);
    lmhead_phase<HS>(c, sm, rg, rs);
    stamp(c, ph, 5, tid == 0);
  }
  if (blockIdx.x == 0) final_phase(c, sm);
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
