// Persistent decode step for gfx950: the whole single-token forward in ONE
// kernel launch, one 512-thread workgroup (8 waves) per CU, all resident.
//
// A decode step is a chain of 5 dependent phases per layer.  As separate
// kernels every dependency costs a launch gap plus the ramp and tail of the
// next kernel; here each dependency is a device-scope handshake instead.
// Producers publish every value as a 64-bit word {f32 value | tag << 32} with
// one relaxed agent-scope store; consumers spin with relaxed agent-scope loads
// until every word carries the tag they expect.  No fences, no shared
// counters, no L2 writeback/invalidate: the tag itself says the value is there.
//
// Roles.  Every CU serves ONE phase kind in every layer (the host sizes the
// five groups of CUs in proportion to their bytes per layer):
//   Q   rows of q|k|v = W_qkv RMSNorm(x0) + b                          -> QKV
//   A   attention item (kv head g, split s): QK-norm, RoPE, KV-cache write,
//       online softmax over its positions; split partials merged        -> O
//   O   rows of x1 = x0 + W_o o                                          -> X1
//   GU  rows of act = SiLU(W_g h2) * (W_u h2), h2 = RMSNorm(x1)           -> ACT
//   D   rows of x0' = x1 + W_d act                                       -> X0
// (tag = seq << 8 | l; D publishes x0' with the tag of layer l + 1.)
// A CU that has finished its phase of layer l has four handshakes of time
// before its input of layer l + 1 can exist, so it loads its whole slice of
// layer l + 1 (weights, or the cached K/V rows of its item) into registers
// right away: the weight stream runs beside the chain of handshakes instead of
// inside it, and each buffer is polled by one group of CUs only.  After the
// last layer every CU loads the first batch of its LM-head rows the same way;
// then all CUs take the final RMSNorm + tied LM head with per-CU argmax
// partials, and CU 0 the argmax over the partials, advancing the step state.
//
// Inputs.  Before polling at full rate a CU watches one word of its
// producer's own input (a gate).  The attention role (and shapes that do not
// form matrix-core tiles) then polls its whole input with all 512 threads
// into LDS, followed by one workgroup barrier.  A matrix-core GEMV role polls
// per wave instead: each wave takes only the input words of its own column
// chunks, so no barrier separates the input from the products.  The SwiGLU
// activations and the attention output travel as value pairs (two values to
// 16 significant bits per word), halving the words those consumers poll.
//
// GEMV on the matrix cores: a role's rows form 16 x 32 bf16 tiles, the input
// enters as the bf16 pair (hi, lo) in two rows of the other operand, and each
// wave accumulates its own column chunks, the 8 partials of a row being added
// in LDS after the one barrier.  RMSNorm is folded in: the LDS input is
// gain * x and each row sum is scaled by 1/RMS(x) afterwards.
//
// The fused QKV rows are stored group-major ([kv head g][q heads of g | k_g |
// v_g] x 128), so one attention item reads one contiguous run.
//
// Reusing a buffer across layers is safe: every reader of a buffer instance
// is, through the dataflow, a required producer of what the next writer of
// that buffer waits for.  This needs every CU of a role to own at least one
// output row (the host plans it so), and every LDS input slot is rewritten
// only after a workgroup barrier that all waves reach after their last read
// of it (slots alternate by layer).

#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "persist.h"

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kSeg = 512;  // bf16 per segment: 64 lanes x 8 values (16 bytes)
constexpr int kBatch = 8;  // segments per wave per streamed batch
constexpr int kFirst = 24; // segments per wave loaded ahead (one layer slice, or the first LM-head rows)
constexpr int D = 128;     // head_dim
constexpr int kVecMax = 11264;
constexpr int kResMax = 512;  // residual rows of one CU (O and D roles)
constexpr int kOutMax = 4096; // output units of one CU in a phase (and LM-head rows)
constexpr int kTraceL = 64;   // layers covered by the phase trace
constexpr int kAttStride = D + 4;  // {m, l, -, -, o[128]}: o stays 16-byte aligned
constexpr int kRedStride = 68;     // row stride of the GEMV row-sum scratch (floats)
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
constexpr int kTokLayer = 254;  // tag "layer" of the token word (unique to that word)

// Positions per attention split at context ctx, as the step plan cuts them:
// splits no longer than the rows a CU loads ahead, on at most half the grid.
__host__ __device__ inline int split_plan(int ctx, int grid, int nkv, int* chunk) {
  const int span = kFirst / 8 * 64;
  const int smax = grid / (2 * nkv);
  int S = (ctx + span - 1) / span;
  S = S < smax ? S : smax;
  const int ch = (ctx + S - 1) / S;
  *chunk = ch;
  return (ctx + ch - 1) / ch;  // every split holds at least one position
}
__device__ __forceinline__ int step_chunk(int ctx, int grid, int nkv) {
  int ch;
  (void)split_plan(ctx, grid, nkv, &ch);
  return ch;
}

// Value pairs: a 64-bit word {tag16 << 48 | a24 << 24 | b24} carries two
// values rounded to 16 significant bits (the top 24 bits of the float, to
// nearest even) for a consumer that multiplies them as bf16 halves anyway, and
// the low 16 bits of the tag (8 bits of the step, the layer).
__device__ __forceinline__ uint64_t f24(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint64_t)((u + 0x7Fu + ((u >> 8) & 1u)) >> 8);
}
__device__ __forceinline__ float unf24(uint64_t b) { return __uint_as_float((uint32_t)(b & 0xFFFFFFu) << 8); }
__device__ __forceinline__ void st_pair(uint64_t* p, float a, float b, uint32_t tag) {
  __hip_atomic_store(gl(p), ((uint64_t)(tag & 0xFFFFu) << 48) | (f24(a) << 24) | f24(b), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

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

struct Smem {
  float vec[2][kVecMax];    // phase inputs (gain * x for normed phases), slot = layer & 1
  float xres[2][kResMax];   // residual rows of this CU, slot = layer & 1
  float att[kWaves * 8 * kAttStride > kWaves * 16 * kRedStride ? kWaves * 8 * kAttStride : kWaves * 16 * kRedStride];
  float qk[10 * D];  // rotated q heads, k, v of one kv group
  float red[48];     // [0, 16): RMS partials by slot; [32, 48): LM-head argmax
  float outv[kOutMax];  // this CU's results of a phase, published together at its end
  uint64_t ts[kTraceL + 2][8];  // phase-trace stamps of this CU's phases (written out at the end)
  int abort_flag;
};

static_assert(sizeof(Smem) <= 160 * 1024, "the workgroup's LDS holds Smem");

enum { kQKV = 0, kAttn = 1, kOproj = 2, kGateUp = 3, kDown = 4 };

struct Ctx {
  const AS4 PersistConst* a;
  int pos, S, chunk, X;  // X: head groups per kv head (attention items = nkv X S)
  float eps;
  uint32_t seq;
  uint64_t t0;
  int role, rank, nrole;  // this CU's role, its index among the CUs of the role, their number
  int r0, r1;             // the role's output units of this CU (rows; gate/up row pairs)
  int v0, v1;             // vocabulary rows of this CU (every CU)
};

// Phase-trace stamps go to LDS (a global store here would make later waits on
// the memory counter also wait for it) and are written out when the step ends.
// Local phase index: layer l, then L (LM head) and L + 1 (final argmax);
// slots 0..5 of the trace layout.
__device__ __forceinline__ void stamp(const Ctx& c, Smem& sm, int ph, int what, bool who) {
  if (c.a->trace && who) {
    const int L = c.a->L;
    const int li = ph < 5 * L ? ph / 5 : L + (ph - 5 * L);
    if (li < kTraceL + 2) sm.ts[li][what] = __builtin_amdgcn_s_memrealtime();
  }
}

__device__ __forceinline__ void trace_flush(const Ctx& c, Smem& sm) {
  const AS4 PersistConst& a = *c.a;
  const int n = (min(a.L, kTraceL) + 2) * 8;
  uint64_t* out = a.trace + (size_t)blockIdx.x * persist_trace_slots(a.L);
  if (threadIdx.x == 0) *gl(out + 7) = c.t0;  // kernel start: phase 0, slot 7
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int li = i / 8, k = i % 8;
    const uint64_t v = sm.ts[li][k];
    if (v == 0) continue;
    const int ph = li < a.L ? 5 * li + c.role : 5 * a.L + (li - a.L);
    *gl(out + ph * kTraceSlots + k) = v;
  }
}

// Workgroup barrier ordering LDS only: the waves wait for their own LDS
// operations, not for global loads still in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ bool timed_out(const Ctx& c) {
  return ld_u32(&c.a->err[0]) != 0 || __builtin_amdgcn_s_memrealtime() - c.t0 > kTimeoutTicks;
}

// ------------------------------------------------------------------ polling
// All 512 threads: copy n tagged values src[0..n) (and n2 <= 512 values
// src2[0..n2) to dst2) into LDS once every tag equals `tag`.  With `gain`, the
// LDS copy is gain[k] * x[k] and *rs receives 1 / sqrt(mean(x^2) + eps), the
// RMSNorm scale, applied to the row sums later.  Ends with a workgroup
// barrier; returns false on every thread when the step is abandoned.  With
// `packed`, src holds n / 2 words of value pairs.
template <int PE = kPE>
__device__ __forceinline__ bool poll(const Ctx& c, Smem& sm, int ph, const uint64_t* src, int n, uint32_t tag, float* dst,
                     const float* gain, float* rs, const uint64_t* src2, int n2, float* dst2,
                     bool packed = false) {
  const int tid = threadIdx.x;
  bool ok = !sm.abort_flag;
  float ss = 0.f;
  if (packed) {  // n / 2 words of value pairs (no gain)
    const int nw = n >> 1;
    const uint32_t t16 = tag & 0xFFFFu;
    for (int base = 0; ok && base < nw; base += PE * kThreads) {
      uint64_t v[PE], v2 = (uint64_t)tag << 32;
      uint32_t spin = 0;
      for (;;) {
        bool done = true;
#pragma unroll
        for (int e = 0; e < PE; ++e) {
          const int w = base + e * kThreads + tid;
          v[e] = w < nw ? ld_tagged(src + w) : (uint64_t)t16 << 48;
        }
        if (base == 0 && tid < n2) v2 = ld_tagged(src2 + tid);
#pragma unroll
        for (int e = 0; e < PE; ++e) done &= (uint32_t)(v[e] >> 48) == t16;
        done &= (uint32_t)(v2 >> 32) == tag;
        if (done) break;
        if ((++spin & 31) == 0 && timed_out(c)) {
          st_u32(&c.a->err[0], 1);
          ok = false;
          break;
        }
      }
      if (!ok) break;
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        const int w = base + e * kThreads + tid;
        if (w < nw) {
          const float x0 = unf24(v[e] >> 24), x1 = unf24(v[e]);
          dst[2 * w] = x0;
          dst[2 * w + 1] = x1;
          ss += x0 * x0 + x1 * x1;
        }
      }
      if (base == 0 && tid < n2) dst2[tid] = __uint_as_float((uint32_t)v2);
    }
  }
  for (int base = 0; ok && !packed && base < n; base += PE * kThreads) {
    float gv[PE];
    if (gain) {
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        const int i = base + e * kThreads + tid;
        gv[e] = i < n ? ld_f(gain + i) : 0.f;
      }
    }
    const uint64_t want = (uint64_t)tag << 32;
    uint64_t v[PE], v2 = want;
    uint32_t spin = 0;
    for (;;) {
      bool done = true;
#pragma unroll
      for (int e = 0; e < PE; ++e) {
        const int i = base + e * kThreads + tid;
        v[e] = i < n ? ld_tagged(src + i) : want;
      }
      if (base == 0 && tid < n2) v2 = ld_tagged(src2 + tid);
#pragma unroll
      for (int e = 0; e < PE; ++e) done &= (uint32_t)(v[e] >> 32) == tag;
      done &= (uint32_t)(v2 >> 32) == tag;
      if (done) break;
      if ((++spin & 31) == 0 && timed_out(c)) {
        st_u32(&c.a->err[0], 1);
        ok = false;
        break;
      }
    }
    if (!ok) break;
#pragma unroll
    for (int e = 0; e < PE; ++e) {
      const int i = base + e * kThreads + tid;
      if (i < n) {
        const float x = __uint_as_float((uint32_t)v[e]);
        const float y = gain ? x * gv[e] : x;
        dst[i] = y;
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
    *rs = rsqrtf(t / (float)n + c.eps);
  }
  return true;
}

// Attention item of an A-role CU: kv head g, head group x (q heads j0 ..
// j0 + gi - 1 of the group), split s.
struct Item {
  int g, x, s, j0, gi;
};
template <int G>
__device__ __forceinline__ Item item_of(const Ctx& c) {
  const int per = c.X * c.S;
  Item it;
  it.g = c.rank / per;
  it.x = (c.rank % per) / c.S;
  it.s = c.rank % c.S;
  it.gi = G / c.X;
  it.j0 = it.x * it.gi;
  return it;
}

// ------------------------------------------------------------ role geometry
// A GEMV role: units [0, nunits) of this CU; unit u belongs to wave u % 8 and
// covers `rpu` rows of K values, read in segments of 512.
struct Gemv {
  const uint16_t* a;  // first row of this CU's slice (gate rows for pairs)
  long delta;         // up rows - gate rows, in elements (pairs only)
  int K, nseg, rpu, nunits;
};

__device__ __forceinline__ Gemv gemv_of(const Ctx& c, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  Gemv g;
  g.delta = 0;
  g.rpu = 1;
  g.nunits = c.r1 - c.r0;
  switch (c.role) {
    case kQKV: g.K = a.H; g.a = L.wqkv; break;
    case kOproj: g.K = a.nq * D; g.a = L.wo; break;
    case kGateUp: g.K = a.H; g.a = L.wg; g.delta = (long)(L.wu - L.wg); g.rpu = 2; break;
    default: g.K = a.I; g.a = L.wd; break;
  }
  g.a += (size_t)c.r0 * g.K;
  g.nseg = (g.K + kSeg - 1) / kSeg;
  return g;
}

// The LoRA-down CU ("EMBERGLASS (qwen-webgpu-lora) README", LoRA sections: a
// live rank-r adapter on q_proj and v_proj): rows [A_q; A_v] of layer l, 2 r
// rows of H, as a row-segment GEMV whose outputs go to QKV[nqkv ..].
__device__ __forceinline__ Gemv lora_of(const Ctx& c, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  Gemv g;
  g.a = L.lora_a;
  g.delta = 0;
  g.K = a.H;
  g.nseg = (a.H + kSeg - 1) / kSeg;
  g.rpu = 1;
  g.nunits = 2 * a.lora_r;
  return g;
}

// Matrix-core geometry of a GEMV role.  The CU's rows (per row set: gate and
// up rows for pairs) form blocks of 16 (the last block shifted back to end at
// the last row, overlapping its neighbour); the K columns form chunks of 32,
// dealt to the 8 waves in pairs (see tile_chunk).  A register
// slot holds one 16 x 32 tile: lane i has row i % 16, columns 8 (i / 16) ..
// + 7.  The tiles of every wave fit in the registers loaded ahead.
struct Tiles {
  int nb;   // row blocks per row set
  int ns;   // row sets: 2 for gate/up pairs, else 1
  int nkw;  // chunks per wave (K / 256)
};

// The j-th chunk of wave w: chunk pairs 2 w, 2 w + 1 (both halves of a row's
// 128-byte line), then 2 w + 16, 2 w + 17, ...
__device__ __forceinline__ int tile_chunk(int w, int j) { return 16 * (j >> 1) + 2 * w + (j & 1); }

__device__ __forceinline__ int gemv_k(const Ctx& c) {
  const AS4 PersistConst& a = *c.a;
  return c.role == kOproj ? a.nq * D : c.role == kDown ? a.I : a.H;
}

// Whether this CU's GEMV role runs on the matrix cores (and so stages its
// input as bf16 halves); the other shapes take the row-segment path.
__device__ __forceinline__ bool mfma_path(const Ctx& c, Tiles* t = nullptr) {
  if (c.role == kAttn) return false;
  const int K = gemv_k(c), n = c.r1 - c.r0;
  Tiles g;
  g.nb = (n + 15) >> 4;
  g.ns = c.role == kGateUp ? 2 : 1;
  g.nkw = K >> 8;
  if (t) *t = g;
  const bool kw = g.nkw == 4 || g.nkw == 6 || g.nkw == 8 || g.nkw == 12;
  return (K & 255) == 0 && kw && n >= 16 && g.ns * g.nb <= 6 && g.ns * g.nb * g.nkw <= kFirst;
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

// ----------------------------------------------------------------- registers
// The slice loaded ahead (weight segments, or the K/V rows of the attention
// item: K in the first half, V in the second) is loaded at ONE program point
// of the layer loop; each role only computes addresses.  Values defined on
// several paths would be merged with register copies, and a copy waits for
// its load.
template <int N>
struct Regs {
  u32x4 R[N];
};

// N loads of 16 bytes per lane from buffer records: slot i reads
// base[i < N/2 ? 0 : 1] + voff + soff[i], where voff is the lane's part and
// soff[i] is wave-uniform (a scalar register), so a batch costs one vector
// register of addressing.  Every byte read lies inside its allocation: the
// uniform offsets stay inside the matrix or cache block, and the lane part of
// a row or position past the end lands in the allocations' tail padding.
template <int N>
struct Addr {
  __amdgpu_buffer_rsrc_t rs[2];
  int voff;
  int soff[N];
  int n = N;  // slots to load (wave-uniform); the others keep stale values and are not used
};

// int4 roles: the slots' fp16 group scales, one per lane and slot (record,
// lane part, uniform parts, count).
template <int N>
struct SAddr {
  __amdgpu_buffer_rsrc_t rs;
  int voff;
  int soff[N];
  int n;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

template <int N>
__device__ __forceinline__ void load_regs(Regs<N>& rg, const Addr<N>& ad) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < ad.n)
      rg.R[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.rs[i < N / 2 ? 0 : 1], ad.voff, ad.soff[i], 2 /* nt */));
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// The group scales of an int4 role's slots (fp16 bit patterns, one per lane
// and slot), into registers sc[H0 ..]; issued beside the codes' loads.
template <int H0, int N, int M>
__device__ __forceinline__ void load_scales(uint32_t (&sc)[M], const SAddr<N>& ad) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i < ad.n) sc[H0 + i] = __builtin_amdgcn_raw_buffer_load_b16(ad.rs, ad.voff, ad.soff[i], 2 /* nt */);
}

// The next N segments from walk position w (the last valid segment repeats
// past the end, so every register is loaded).  A row's last segment may run
// past K: those lanes read the next row or the padding, and the dot product
// skips them.
template <int N>
__device__ __forceinline__ void gemv_addr(Addr<N>& ad, const Gemv& g, Walk w) {
  ad.rs[0] = ad.rs[1] = rsrc_of(g.a);
  ad.voff = (int)(threadIdx.x & 63) * 16;
  Walk last = w;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (walk_valid(g, w)) last = w;
    ad.soff[i] = (int)(((long)last.t * g.delta + (long)min(last.u, g.nunits - 1) * g.K + last.sg * kSeg) * 2);
    walk_next(g, w);
  }
}

// The tiles of this wave (see Tiles): slot bb nkw + j holds row block bb (row
// set bb / nb) and chunk tile_chunk(wave, j); slots past the tiles are not loaded.
// Every row read lies inside the CU's own rows.
template <int N>
__device__ __forceinline__ void tile_addr(Addr<N>& ad, const Gemv& g, const Tiles& t, int nrows) {
  ad.rs[0] = ad.rs[1] = rsrc_of(g.a);
  const int lane = threadIdx.x & 63, wave = wave_id();
  ad.voff = (lane & 15) * g.K * 2 + (lane >> 4) * 16;
  const int T = t.ns * t.nb * t.nkw;
  ad.n = T;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int ii = min(i, T - 1);
    const int bb = ii / t.nkw, j = ii - bb * t.nkw;
    const int set = bb / t.nb, b = bb - set * t.nb;
    const int row = min(16 * b, nrows - 16);
    ad.soff[i] = (int)(((long)set * g.delta + (long)row * g.K + tile_chunk(wave, j) * 32) * 2);
  }
}

// Attention steps t0 .. t0 + N/8 - 1: lane q8 of group pg reads dims
// 32 k + 4 q8 .. + 3 (k < 4) of position p_begin + 64 t + 8 wave + pg; K
// fragment k of step t in slot 4 t + k, V in N/2 + 4 t + k.  Positions past the
// split are read (inside the cache block or its padding) and not used.
template <int N>
__device__ __forceinline__ void kv_addr(Addr<N>& ad, const float* Kg, const float* Vg, int p_begin, int t0) {
  ad.rs[0] = rsrc_of(Kg);
  ad.rs[1] = rsrc_of(Vg);
  ad.voff = (int)((threadIdx.x & 63) >> 3) * D * 4 + (int)(threadIdx.x & 7) * 16;
  const int p0 = p_begin + 8 * wave_id();
#pragma unroll
  for (int t = 0; t < N / 8; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int off = (p0 + 64 * (t0 + t)) * D * 4 + k * 128;
      ad.soff[4 * t + k] = off;
      ad.soff[N / 2 + 4 * t + k] = off;
    }
  }
}

// LM head: rows rb, rb + 8, ... (N / HS rows of HS segments) of this CU's
// vocabulary slice E (first row), clamped into it.
template <int N, int HS>
__device__ __forceinline__ void lm_addr(Addr<N>& ad, const uint16_t* E, int rb, int nrows) {
  ad.rs[0] = ad.rs[1] = rsrc_of(E);
  ad.voff = (int)(threadIdx.x & 63) * 16;
#pragma unroll
  for (int i = 0; i < N / HS; ++i) {
    const int rr = min(rb + i * kWaves, nrows - 1);
#pragma unroll
    for (int sg = 0; sg < HS; ++sg) ad.soff[i * HS + sg] = (rr * HS + sg) * kSeg * 2;
  }
}

// ---------------------------------------------------------- int4 GEMV roles
// A role's rows in int4 group-128 form (codes u8 [rows][K / 2], byte b of a
// row = columns 2b (low nibble) and 2b + 1 (high nibble) as code + 8; fp16
// scales [rows][K / 128]) are read in slots of one 16-row block by one group
// of 128 columns: lane i loads the 16 bytes of row i % 16, columns
// 32 (i / 16) .. + 31, and one scale (its row's, of the slot's group).  Groups
// are dealt to the waves round robin (wave w: groups w, w + 8, ...); a wave's
// slots run row block by row block, its groups inner.  The first kFirst slots
// are loaded a layer ahead, the rest stream in during the phase.
struct Q4Geo {
  const uint8_t* c;   // codes of the CU's first row (gate rows for pairs)
  const uint16_t* s;  // scales of the CU's first row
  int dc, ds;         // up rows - gate rows: codes (bytes), scales (elements)
  int K, ng;          // columns, groups of 128
  int nb, ns, nrows;  // row blocks per row set, row sets, rows per set
  int cnt, nslots;    // groups and slots of this wave
};

__device__ __forceinline__ Q4Geo q4_geo(const Ctx& c, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& L = ((const AS4 LayerPtrs*)a.layers)[l];
  Q4Geo q;
  // the projection of the role (q|k|v 0, o 1, gate/up 2, down 3), selected by
  // index rather than by a branch per role
  const int p = c.role - (c.role > kAttn ? 1 : 0);
  q.c = L.qcode[p];
  q.s = L.qscale[p];
  q.K = c.role == kOproj ? a.nq * D : c.role == kDown ? a.I : a.H;
  q.ns = c.role == kGateUp ? 2 : 1;
  q.dc = c.role == kGateUp ? a.I * (a.H >> 1) : 0;
  q.ds = c.role == kGateUp ? a.I * (a.H >> 7) : 0;
  q.ng = q.K >> 7;
  q.nrows = c.r1 - c.r0;
  q.nb = (q.nrows + 15) >> 4;
  q.c += (size_t)c.r0 * (q.K >> 1);
  q.s += (size_t)c.r0 * q.ng;
  const int w = wave_id();
  q.cnt = __builtin_amdgcn_readfirstlane(w < q.ng ? (q.ng - 1 - w) / kWaves + 1 : 0);
  q.nslots = __builtin_amdgcn_readfirstlane(q.ns * q.nb * q.cnt);
  return q;
}

// Addresses of this wave's slots i0 .. i0 + N - 1 (those past its last slot
// are not loaded).  Every row read lies inside the CU's own rows.
// Row block and group of the wave's slot ii: {set, first row, group}.
struct Q4Slot {
  int set, row, g;
};
__device__ __forceinline__ Q4Slot q4_slot_of(const Q4Geo& q, int ii) {
  const int cnt = max(q.cnt, 1);
  const int bb = ii / cnt, j = ii - bb * cnt;
  Q4Slot t;
  t.set = bb / q.nb;
  t.row = min(16 * (bb - t.set * q.nb), q.nrows - 16);
  t.g = wave_id() + kWaves * j;
  return t;
}

template <int N>
__device__ __forceinline__ void q4_addr(Addr<N>& ad, const Q4Geo& q, int i0) {
  const int lane = threadIdx.x & 63;
  const int n = max(0, min(N, q.nslots - i0));
  ad.rs[0] = ad.rs[1] = rsrc_of(q.c);
  ad.voff = (lane & 15) * (q.K >> 1) + (lane >> 4) * 16;
  ad.n = n;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const Q4Slot t = q4_slot_of(q, i0 + min(i, max(n - 1, 0)));
    ad.soff[i] = __builtin_amdgcn_readfirstlane(t.set * q.dc + t.row * (q.K >> 1) + t.g * 64);  // wave-uniform
  }
}

template <int N>
__device__ __forceinline__ void q4_saddr(SAddr<N>& sa, const Q4Geo& q, int i0) {
  const int lane = threadIdx.x & 63;
  const int n = max(0, min(N, q.nslots - i0));
  sa.rs = rsrc_of(q.s);
  sa.voff = (lane & 15) * q.ng * 2;
  sa.n = n;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const Q4Slot t = q4_slot_of(q, i0 + min(i, max(n - 1, 0)));
    sa.soff[i] = __builtin_amdgcn_readfirstlane((t.set * q.ds + t.row * q.ng + t.g) * 2);
  }
}

// K and V cache rows of (layer l, kv head g).
__device__ __forceinline__ float* k_rows(const AS4 PersistConst& a, int l, int g) {
  return a.Kc + ((size_t)l * a.nkv + g) * a.max_pos * D;
}
__device__ __forceinline__ float* v_rows(const AS4 PersistConst& a, int l, int g) {
  return a.Vc + ((size_t)l * a.nkv + g) * a.max_pos * D;
}

// The slice this CU loads ahead for layer l (l == L: its first LM-head rows).
template <int HS, bool Q4, bool LORA>
__device__ __forceinline__ Addr<kFirst> ahead_addr(const Ctx& c, int l, bool lora) {
  const AS4 PersistConst& a = *c.a;
  const int wave = wave_id();
  Addr<kFirst> ad;
  if (l >= a.L) {
    lm_addr<kFirst, HS>(ad, a.embed + (size_t)c.v0 * HS * kSeg, wave, c.v1 - c.v0);
  } else if (c.role == kAttn) {
    const int g = c.rank / (c.X * c.S), s = c.rank % c.S;
    kv_addr<kFirst>(ad, k_rows(a, l, g), v_rows(a, l, g), s * c.chunk, 0);
  } else if (LORA && lora) {
    gemv_addr<kFirst>(ad, lora_of(c, l), Walk{wave, 0, 0});
  } else if (Q4) {
    q4_addr<kFirst>(ad, q4_geo(c, l), 0);
  } else {
    Tiles t;
    if (mfma_path(c, &t))
      tile_addr<kFirst>(ad, gemv_of(c, l), t, c.r1 - c.r0);
    else
      gemv_addr<kFirst>(ad, gemv_of(c, l), Walk{wave, 0, 0});
  }
  return ad;
}

// ------------------------------------------------------------------- phases
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kTileRed = 96;  // tile rows a CU's partials cover (6 blocks of 16 rows)

// GEMV tiles on the matrix cores (see Tiles).  Each 16 x 16 x 32 product takes
// one input chunk of the wave as operand A, whose rows 0 and 1 are the bf16
// halves hi and lo of the 32 inputs (the other rows are not used), and one
// weight tile as operand B; result rows 0 and 1 of lane n < 16 accumulate row
// n of the block against hi and lo.  Lanes 0..15 then write each block's
// partial (hi + lo over the wave's chunks) to LDS.
template <int NKW, int NBT>
__device__ __forceinline__ void gemv_tiles(const Ctx& c, Smem& sm, const Regs<kFirst>& rg, const float* h, int l) {
  static_assert(NKW * NBT <= kFirst && NBT * 16 <= kTileRed, "tiles fit the registers and the LDS partials");
  static_assert(kTileRed * kWaves <= sizeof(Smem::att) / sizeof(float), "the partials fit the scratch");
  const int lane = threadIdx.x & 63, wave = wave_id();
  u32x4 xa[NKW];
#pragma unroll
  for (int j = 0; j < NKW; ++j)  // 8 inputs as hi[8] then lo[8]: lane 1 of each 16 takes the lo half
    xa[j] = *reinterpret_cast<const u32x4*>(h + tile_chunk(wave, j) * 32 + (lane >> 4) * 8 + ((lane & 15) == 1 ? 4 : 0));
  __builtin_amdgcn_sched_barrier(0);  // every LDS read in flight before the first product
  f32x4 acc[NBT];
#pragma unroll
  for (int bb = 0; bb < NBT; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NKW; ++j)
#pragma unroll
    for (int bb = 0; bb < NBT; ++bb)
      acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[j]),
                                                        __builtin_bit_cast(bf16x8_t, rg.R[bb * NKW + j]), acc[bb], 0, 0, 0);
  stamp(c, sm, 5 * l + c.role, 6, threadIdx.x == 0);
  if (lane < 16) {  // partial of row bb * 16 + lane at [row][wave]: a row's 8 partials are contiguous
#pragma unroll
    for (int bb = 0; bb < NBT; ++bb) sm.att[(bb * 16 + lane) * kWaves + wave] = acc[bb].x + acc[bb].y;
  }
}

__device__ __forceinline__ void gemv_tiles_any(const Ctx& c, Smem& sm, const Tiles& t, const Regs<kFirst>& rg,
                                               const float* h, int l) {
#define QD_TILES(K, B) \
  case K * 8 + B: gemv_tiles<K, B>(c, sm, rg, h, l); break;
  switch (t.nkw * 8 + t.ns * t.nb) {
    QD_TILES(4, 1) QD_TILES(4, 2) QD_TILES(4, 3) QD_TILES(4, 4) QD_TILES(4, 5) QD_TILES(4, 6)
    QD_TILES(6, 1) QD_TILES(6, 2) QD_TILES(6, 3) QD_TILES(6, 4)
    QD_TILES(8, 1) QD_TILES(8, 2) QD_TILES(8, 3)
    QD_TILES(12, 1) QD_TILES(12, 2)
    default: break;  // excluded by mfma_path
  }
#undef QD_TILES
}

// Output row u of a GEMV role: publishing is every unit at once, one word
// per thread, so a wave's stores cover whole cache lines (single-word stores
// spread over lines reach the pollers much later).
__device__ __forceinline__ void publish_row(const Ctx& c, Smem& sm, int l, int u, float t, const float* bias) {
  const AS4 PersistConst& a = *c.a;
  const float* xr = sm.xres[l & 1];
  const int r = c.r0 + u;
  switch (c.role) {
    case kQKV: st_tagged(a.QKV + r, bias ? t + ld_f(bias + r) : t, tag_of(c.seq, l)); break;
    case kOproj: st_tagged(a.X1 + r, xr[u] + t, tag_of(c.seq, l)); break;
    default: st_tagged(a.X0 + r, xr[u] + t, tag_of(c.seq, l + 1)); break;
  }
}

// Matrix-core GEMV, after the barrier that follows the products: unit u sums
// the 8 waves' partials of its row (and of its up row for pairs) and
// publishes.
__device__ __forceinline__ void tiles_finish(const Ctx& c, Smem& sm, int l, const Tiles& tl, float rs, const float* bias) {
  const AS4 PersistConst& a = *c.a;
  const int kind = c.role;
  const uint32_t tag = tag_of(c.seq, l);
  {
    const int nrows = c.r1 - c.r0;
    auto sum8 = [&](int row) {  // the 8 wave partials of a tile row, in a fixed order
      const f32x4 p = *reinterpret_cast<const f32x4*>(sm.att + row * kWaves);
      const f32x4 q = *reinterpret_cast<const f32x4*>(sm.att + row * kWaves + 4);
      return ((p.x + p.y) + (p.z + p.w)) + ((q.x + q.y) + (q.z + q.w));
    };
    auto unit = [&](int u) {
      const int b = min(u >> 4, tl.nb - 1);
      const int n = b * 16 + u - min(16 * b, nrows - 16);
      float t = sum8(n) * rs;
      if (tl.ns == 2) t = sum8(tl.nb * 16 + n) * rs * t * __builtin_amdgcn_rcpf(1.0f + __expf(-t));  // up * SiLU(gate)
      return t;
    };
    if (kind == kGateUp) {  // value pairs (the CU's units start at an even unit)
      for (int u = 2 * threadIdx.x; u < nrows; u += 2 * kThreads) st_pair(a.ACT + ((c.r0 + u) >> 1), unit(u), unit(u + 1), tag);
    } else {
      for (int u = threadIdx.x; u < nrows; u += kThreads) publish_row(c, sm, l, u, unit(u), bias);
    }
    stamp(c, sm, 5 * l + kind, 2, threadIdx.x == 0);
  }
}

// int4 roles' input as int8 pieces for the matrix cores.  The phase input h
// (f32, gain * x for normed phases) over the wave's groups (128 columns each;
// group g belongs to wave g % 8) is written as y = u (a + b / 128 + c / 16384)
// with one power of two u per wave (its largest |y| lies in [64 u, 128 u)),
// a = trunc(y / u), b and c the next seven-bit digits (c rounded to nearest):
// |error| <= u / 32768, i.e. 2^-21 of the wave's largest input.  The pieces
// a, b, c go to rows 0, 4 and 8 of the A operand of v_mfma_i32_16x16x64_i8, so
// the three products land in lanes 0-15, 16-31 and 32-47 of one result; the
// other rows read a record of zeros after the groups.  LDS layout per group:
// [parity e][piece p][quarter q][16 bytes], byte 4 m + t of quarter q being
// column 128 g + 32 q + 8 m + 2 t + e (the order in which the codes' nibbles
// unpack).  Each 16-lane team of a wave converts one of the wave's groups
// (lane: quarter q, dword m).  Returns u / 16 (the codes enter as 16 code).
constexpr int kQ4Group = 384;  // LDS bytes of one group's pieces

__device__ __forceinline__ float q4_stage(const float* h, uint8_t* q8, const Q4Geo& q) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = lane >> 4, l16 = lane & 15, qq = l16 >> 2, m = l16 & 3;
  float mx = 0.f;  // the wave's largest |y|
  for (int j0 = 0; j0 < q.cnt; j0 += 4) {  // wave-uniform
    const int j = j0 + t;
    if (j < q.cnt) {
      const int col = 128 * (wave + kWaves * j) + 32 * qq + 8 * m;
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(h + col);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(h + col + 4);
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(y0.x), fabsf(y0.y)), fmaxf(fabsf(y0.z), fabsf(y0.w))));
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(y1.x), fabsf(y1.y)), fmaxf(fabsf(y1.z), fabsf(y1.w))));
    }
  }
  mx = wave_max(mx);
  const int E = (int)((__float_as_uint(mx) >> 23) & 0xFF);  // mx in [2^(E-127), 2^(E-126))
  const bool live = E >= 6;  // inputs below 2^-121 (or all zero) are taken as zero
  const float up = __uint_as_float((uint32_t)(live ? 260 - E : 127) << 23);  // 1 / u = 2^(133 - E)
  for (int j0 = 0; j0 < q.cnt; j0 += 4) {  // wave-uniform
    const int j = j0 + t;
    if (j >= q.cnt) continue;
    const int g = wave + kWaves * j;
    const int col = 128 * g + 32 * qq + 8 * m;
    const f32x4 y0 = *reinterpret_cast<const f32x4*>(h + col);
    const f32x4 y1 = *reinterpret_cast<const f32x4*>(h + col + 4);
    const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
    uint32_t pk[6] = {0u, 0u, 0u, 0u, 0u, 0u};  // [parity][piece]
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float v = live ? y[k] * up : 0.f;  // |v| < 128, exact
      const float a = truncf(v);
      const float r = (v - a) * 128.0f;
      const float b = truncf(r);
      const float cc = fminf(fmaxf(rintf((r - b) * 128.0f), -127.0f), 127.0f);
      const int sh = 8 * (k >> 1), e3 = 3 * (k & 1);
      pk[e3 + 0] |= ((uint32_t)(int)a & 0xFFu) << sh;
      pk[e3 + 1] |= ((uint32_t)(int)b & 0xFFu) << sh;
      pk[e3 + 2] |= ((uint32_t)(int)cc & 0xFFu) << sh;
    }
    uint8_t* d = q8 + g * kQ4Group + qq * 16 + m * 4;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      *reinterpret_cast<uint32_t*>(d + p * 64) = pk[p];
      *reinterpret_cast<uint32_t*>(d + 192 + p * 64) = pk[3 + p];
    }
  }
  if (lane < kQ4Group / 16)  // the record of zeros read by the A rows that hold no piece
    reinterpret_cast<u32x4*>(q8 + q.ng * kQ4Group)[lane] = u32x4{0u, 0u, 0u, 0u};
  return live ? ldexpf(1.0f, E - 137) : 0.f;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// int4 GEMV role: stage the pieces, then every slot of the wave in the order
// (row block, group) (the registers loaded ahead, then streamed halves of
// kFirst / 2 slots, each half reloaded as soon as it is consumed).  A slot is
// two int8 products (even and odd columns of the group: the code nibbles
// become 16 code in the bytes' high halves, exact) into one integer result,
// which, scaled by the slot's group scale, joins a per-lane f32 sum one slot
// later, so that the products' latency hides behind the next slot's work.
// At the end of each row block the three piece sums are weighted (1, 2^-7,
// 2^-14, times the wave's u / 16) and added across lanes in a fixed order,
// and lanes 0-15 leave the wave's partial of each row in LDS for
// tiles_finish.
__device__ __forceinline__ void q4_phase(const Ctx& c, Smem& sm, int l, Regs<kFirst>& rg, uint32_t (&sc)[kFirst],
                                         float rs, const float* bias) {
  const Q4Geo q = q4_geo(c, l);
  const int lane = threadIdx.x & 63, wave = wave_id();
  uint8_t* q8 = reinterpret_cast<uint8_t*>(sm.vec[(l + 1) & 1]);  // the slot of the previous layer's input
  const float u16 = q4_stage(sm.vec[l & 1], q8, q);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads back its own pieces
  const int l16 = lane & 15;
  const bool plane = (l16 & 3) == 0 && l16 < 12;  // A rows 0, 4, 8 hold the pieces
  // A of the wave's group j at a0 + j astep (even columns; odd at + 192); the
  // other rows read the record of zeros after the groups
  const int a0 = plane ? wave * kQ4Group + (l16 >> 2) * 64 + (lane >> 4) * 16 : q.ng * kQ4Group;
  const int astep = plane ? kWaves * kQ4Group : 0;
  const float pw = (lane < 16 ? 1.0f : lane < 32 ? 0.0078125f : lane < 48 ? 6.103515625e-05f : 0.0f) * u16;
  const int nbb = q.ns * q.nb, cnt = max(q.cnt, 1);
  int sb = 0, sj = 0;  // row block and group of the next slot
  float tot = 0.f, ps = 0.f;
  int cur = 0;
  i32x4 pp = {0, 0, 0, 0};  // the previous slot's result (scale ps)
  auto flush = [&]() {
    const float v = tot * pw;
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float v2 = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
    const float v4 = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    if (lane < 16) sm.att[(cur * 16 + lane) * kWaves + wave] = v4;
    tot = 0.f;
    ++cur;
  };
  auto slot = [&](const u32x4 w, uint32_t s16) {
    const int bb = sb, j = sj;
    if (++sj == cnt) {  // wave-uniform cursor of the next slot
      sj = 0;
      ++sb;
    }
    const int aa = a0 + j * astep;
    const u32x4 ae = *reinterpret_cast<const u32x4*>(q8 + aa);
    const u32x4 ao = *reinterpret_cast<const u32x4*>(q8 + aa + 192);
    u32x4 be, bo;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      be[k] = ((w[k] << 4) ^ 0x88888880u) & 0xF0F0F0F0u;
      bo[k] = (w[k] ^ 0x88888888u) & 0xF0F0F0F0u;
    }
    i32x4 acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, ae), __builtin_bit_cast(i32x4, be),
                                                      i32x4{0, 0, 0, 0}, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, ao), __builtin_bit_cast(i32x4, bo), acc, 0, 0,
                                                0);
    tot = fmaf((float)pp.x, ps, tot);  // the previous slot (its products are ready by now)
    while (cur < bb) flush();  // wave-uniform
    pp = acc;
    ps = __half2float(__ushort_as_half((uint16_t)s16));
  };
  constexpr int HN = kFirst / 2;
  for (int base = 0; base < q.nslots; base += kFirst) {  // wave-uniform
#pragma unroll
    for (int r = 0; r < HN; ++r)
      if (base + r < q.nslots) slot(rg.R[r], sc[r]);
    if (base + kFirst < q.nslots) {
      Addr<HN> ad;
      SAddr<HN> sa;
      q4_addr<HN>(ad, q, base + kFirst);
      q4_saddr<HN>(sa, q, base + kFirst);
#pragma unroll
      for (int i = 0; i < HN; ++i)
        if (i < ad.n)
          rg.R[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.rs[0], ad.voff, ad.soff[i], 2));
      load_scales<0>(sc, sa);
    }
#pragma unroll
    for (int r = 0; r < HN; ++r)
      if (base + HN + r < q.nslots) slot(rg.R[HN + r], sc[HN + r]);
    if (base + kFirst + HN < q.nslots) {
      Addr<HN> ad;
      SAddr<HN> sa;
      q4_addr<HN>(ad, q, base + kFirst + HN);
      q4_saddr<HN>(sa, q, base + kFirst + HN);
#pragma unroll
      for (int i = 0; i < HN; ++i)
        if (i < ad.n)
          rg.R[HN + i] =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad.rs[0], ad.voff, ad.soff[i], 2));
      load_scales<HN>(sc, sa);
    }
  }
  tot = fmaf((float)pp.x, ps, tot);
  while (cur < nbb) flush();
  stamp(c, sm, 5 * l + c.role, 2, threadIdx.x == 0);
  __syncthreads();
  tiles_finish(c, sm, l, Tiles{q.nb, q.ns, 0}, rs, bias);
}

// GEMV role: this CU's rows, from the registers loaded ahead (and, on the
// row-segment path, streamed batches for any rest), published one word per
// output row.
template <bool Q4>
__device__ __forceinline__ void gemv_phase(const Ctx& c, Smem& sm, int l, Regs<kFirst>& rg, uint32_t (&sc)[kFirst],
                                           float rs, const Gemv& g, const float* bias) {
  const AS4 PersistConst& a = *c.a;
  const int lane = threadIdx.x & 63, wave = wave_id(), kind = c.role;
  const float* h = sm.vec[l & 1];
  const uint32_t tag = tag_of(c.seq, l);
  stamp(c, sm, 5 * l + kind, 4, threadIdx.x == 0);
  if (Q4) {
    q4_phase(c, sm, l, rg, sc, rs, bias);
    return;
  }
  Tiles tl;
  if (mfma_path(c, &tl)) {
    gemv_tiles_any(c, sm, tl, rg, h, l);
    __syncthreads();
    tiles_finish(c, sm, l, tl, rs, bias);
    return;
  }
  Walk w{wave, 0, 0};
  float acc = 0.f, first = 0.f;
  auto consume = [&](const auto& r, auto n) {
#pragma unroll
    for (int i = 0; i < decltype(n)::value; ++i) {
      if (walk_valid(g, w)) {  // wave-uniform
        const int k = w.sg * kSeg + lane * 8;
        if (k < g.K) acc += dot8(r.R[i], h + k);
        if (w.sg + 1 == g.nseg) {  // row finished
          const float t = wave_total(acc) * rs;
          acc = 0.f;
          if (w.t + 1 < g.rpu) {
            first = t;  // gate row of a pair
          } else if (lane == 0) {
            sm.outv[w.u] = kind == kGateUp ? t * first * __builtin_amdgcn_rcpf(1.0f + __expf(-first)) : t;
          }
        }
        walk_next(g, w);
      }
    }
  };
  consume(rg, std::integral_constant<int, kFirst>{});
  while (walk_valid(g, w)) {  // a slice larger than the registers loaded ahead
    Addr<kBatch> ad;
    gemv_addr<kBatch>(ad, g, w);
    Regs<kBatch> r2;
    load_regs(r2, ad);
    consume(r2, std::integral_constant<int, kBatch>{});
  }
  stamp(c, sm, 5 * l + kind, 2, threadIdx.x == 0);
  __syncthreads();
  if (kind == kGateUp) {
    for (int u = 2 * threadIdx.x; u < g.nunits; u += 2 * kThreads)
      st_pair(a.ACT + ((c.r0 + u) >> 1), sm.outv[u], sm.outv[u + 1], tag);
  } else {
    for (int u = threadIdx.x; u < g.nunits; u += kThreads) publish_row(c, sm, l, u, sm.outv[u], bias);
  }
}

// Matrix-core GEMV role with a per-wave input (QKV from layer 1, o_proj,
// gate/up, down): no workgroup barrier between the poll and the products.
// Every wave watches its own gate word, polls only the input words of its
// column chunks (value pairs for o_proj and down, f32 for the normed QKV and
// gate/up inputs), stages them as bf16 halves for its own A operands and
// multiplies; it also polls its share of the residual rows and keeps its part
// of the input's sum of squares.  One barrier, then the rows are finished.
// Returns false when the step is abandoned.
constexpr int kWE = 6;  // input words per lane at most (12 chunks of 32 f32 values over 64 lanes)

// LoRA-down CU: u = rs [A_q; A_v] (gain * x), 2 r rows from the registers
// loaded ahead (row u on wave u % 8, its segments in slot order), published
// with the layer's tag after the q|k|v rows, where the attention items poll
// them beside their q|k|v.
__device__ __forceinline__ void lora_phase(const Ctx& c, Smem& sm, int l, const Regs<kFirst>& rg, float rs) {
  const AS4 PersistConst& a = *c.a;
  const Gemv g = lora_of(c, l);
  const int lane = threadIdx.x & 63;
  const float* h = sm.vec[l & 1];
  Walk w{wave_id(), 0, 0};
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kFirst; ++i) {
    if (walk_valid(g, w)) {  // wave-uniform
      const int k = w.sg * kSeg + lane * 8;
      if (k < g.K) acc += dot8(rg.R[i], h + k);
      if (w.sg + 1 == g.nseg) {
        const float t = wave_total(acc) * rs;
        acc = 0.f;
        if (lane == 0) sm.outv[w.u] = t;
      }
      walk_next(g, w);
    }
  }
  stamp(c, sm, 5 * l + kQKV, 2, threadIdx.x == 0);
  __syncthreads();
  const uint32_t tag = tag_of(c.seq, l);
  for (int u = threadIdx.x; u < g.nunits; u += kThreads) st_tagged(a.QKV + a.nqkv + u, sm.outv[u], tag);
}

__device__ __forceinline__ bool gemv_waves(const Ctx& c, Smem& sm, int l, const Regs<kFirst>& rg, const Tiles& tl,
                                           const float* bias) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const int lane = threadIdx.x & 63, wave = wave_id(), kind = c.role, nrows = c.r1 - c.r0;
  const uint32_t tag = tag_of(c.seq, l), t16 = tag & 0xFFFFu;
  float* h = sm.vec[l & 1];
  float* xr = sm.xres[l & 1];
  const uint64_t* src;
  const uint64_t* gw;
  const float* gain = nullptr;
  const uint64_t* src2 = nullptr;
  uint32_t gt = tag;
  bool packed = true, gpk = false;
  switch (kind) {
    case kQKV: src = a.X0; gain = Lw.attn_norm; packed = false; gw = a.X1; gt = tag_of(c.seq, l - 1); break;
    case kOproj: src = a.O; gw = a.QKV; if (l > 0) src2 = a.X0 + c.r0; break;
    case kGateUp: src = a.X1; gain = Lw.mlp_norm; packed = false; gw = a.O; gpk = true; break;
    default: src = a.ACT; gw = a.X1; src2 = a.X1 + c.r0; break;
  }
  if (kind == kOproj && l == 0)  // layer 0: the residual is the embedding row
    for (int r = threadIdx.x; r < nrows; r += kThreads) xr[r] = bf16_to_f(*gl(a.embed + (size_t)gl(a.st)->token * a.H + c.r0 + r));
  bool ok = true;
  if (lane == 0) {  // the wave's gate (the other lanes wait for lane 0)
    uint32_t spin = 0;
    for (;;) {
      const uint64_t v = ld_tagged(gw);
      if (gpk ? (int16_t)(uint16_t)((uint32_t)(v >> 48) - gt) >= 0 : (int32_t)((uint32_t)(v >> 32) - gt) >= 0) break;
      if ((++spin & 3) == 0 && timed_out(c)) {
        st_u32(&c.a->err[0], 1);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(32);
    }
  }
  ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
  // the wave's words: q = 64 e + lane < W; chunk j = q / per, word per * tile_chunk(wave, j) + q % per
  const int per = packed ? 16 : 32, W = tl.nkw * per;
  int widx[kWE];
  float gv[kWE];
#pragma unroll
  for (int e = 0; e < kWE; ++e) {
    const int q = 64 * e + lane;
    widx[e] = q < W ? per * tile_chunk(wave, q / per) + q % per : -1;
    gv[e] = gain && widx[e] >= 0 ? ld_f(gain + widx[e]) : 1.f;
  }
  const int ri = wave * 64 + lane;  // residual row of this thread (rows per CU <= 512)
  const bool has2 = src2 && ri < nrows;
  uint64_t v[kWE], v2 = 0;
  uint32_t spin = 0;
  while (ok) {
    bool done = true;
#pragma unroll
    for (int e = 0; e < kWE; ++e) {
      if (widx[e] >= 0) {
        v[e] = ld_tagged(src + widx[e]);
        done &= packed ? (uint32_t)(v[e] >> 48) == t16 : (uint32_t)(v[e] >> 32) == tag;
      }
    }
    if (has2) {
      v2 = ld_tagged(src2 + ri);
      done &= (uint32_t)(v2 >> 32) == tag;
    }
    if (__all(done)) break;
    if ((++spin & 31) == 0 && timed_out(c)) {
      st_u32(&c.a->err[0], 1);
      ok = false;
    }
  }
  float ss = 0.f;
  if (ok) {
#pragma unroll
    for (int e = 0; e < kWE; ++e) {
      if (widx[e] < 0) continue;
      if (packed) {  // values 2w, 2w + 1: adjacent halves of the same 8-value block
        // 16 significant bits: hi = the top 16 bits, lo = x - hi, both exact in bf16
        const int w = widx[e];
        const uint32_t u0 = (uint32_t)((v[e] >> 24) & 0xFFFFFFu) << 8, u1 = (uint32_t)(v[e] & 0xFFFFFFu) << 8;
        const uint32_t l0 = __float_as_uint(__uint_as_float(u0) - __uint_as_float(u0 & 0xFFFF0000u));
        const uint32_t l1 = __float_as_uint(__uint_as_float(u1) - __uint_as_float(u1 & 0xFFFF0000u));
        uint32_t* d = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(h) + (w >> 2) * 16 + ((2 * w) & 7));
        d[0] = (u0 >> 16) | (u1 & 0xFFFF0000u);
        d[4] = (l0 >> 16) | (l1 & 0xFFFF0000u);
      } else {  // bf16 halves of gain * x: hi[8] then lo[8] per 8 values (hi truncated, lo rounded)
        const int i = widx[e];
        const float x = __uint_as_float((uint32_t)v[e]);
        const float y = x * gv[e];
        uint16_t* d = reinterpret_cast<uint16_t*>(h) + (i >> 3) * 16 + (i & 7);
        const uint32_t hb = __float_as_uint(y) >> 16;
        d[0] = (uint16_t)hb;
        d[8] = (uint16_t)bf16_rne(y - __uint_as_float(hb << 16));
        ss += x * x;
      }
    }
    if (has2) xr[ri] = __uint_as_float((uint32_t)v2);
  } else {
    sm.abort_flag = 1;
  }
  stamp(c, sm, 5 * l + kind, 1, threadIdx.x == 0);
  Tiles t2 = tl;
  if (ok) gemv_tiles_any(c, sm, t2, rg, h, l);
  const float wsum = wave_total(ss);
  if (lane == 0) sm.red[((5 * l + kind) & 1) * 8 + wave] = wsum;
  __syncthreads();
  if (sm.abort_flag) return false;
  float rs = 1.f;
  if (gain) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) t += sm.red[((5 * l + kind) & 1) * 8 + i];
    rs = rsqrtf(t / (float)a.H + c.eps);
  }
  tiles_finish(c, sm, l, tl, rs, bias);
  return true;
}

// The attention item's per-lane constants that do not depend on the phase
// input (RoPE row of the position, QK-norm gains): loaded before the input
// poll, so their latency hides behind the handshake.
struct AttnPre {
  float ct, st, gq0, gq1, gk0, gk1;
};
__device__ __forceinline__ AttnPre attn_pre(const Ctx& c, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const int lane = threadIdx.x & 63;
  AttnPre p;
  p.ct = ld_f(a.rope_cos + (size_t)c.pos * (D / 2) + lane);
  p.st = ld_f(a.rope_sin + (size_t)c.pos * (D / 2) + lane);
  p.gq0 = Lw.q_norm ? ld_f(Lw.q_norm + lane) : 1.f;
  p.gq1 = Lw.q_norm ? ld_f(Lw.q_norm + lane + 64) : 1.f;
  p.gk0 = Lw.k_norm ? ld_f(Lw.k_norm + lane) : 1.f;
  p.gk1 = Lw.k_norm ? ld_f(Lw.k_norm + lane + 64) : 1.f;
  return p;
}

// With an adapter: the attention item's LoRA up rows, copied to LDS before
// the input poll (the phase inputs' slots are free in the attention role):
// B_q rows of the item's gi q heads [gi D][r], then B_v rows of its kv head
// [D][r], bf16.
template <int G>
__device__ __forceinline__ void lora_stage(const Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const Item it = item_of<G>(c);
  const int r = a.lora_r;
  const int nq16 = it.gi * D * r / 8, nv16 = D * r / 8;  // 16-byte pieces (D r is a multiple of 8)
  const u32x4* bq = reinterpret_cast<const u32x4*>(Lw.lora_bq + (size_t)(it.g * G + it.j0) * D * r);
  const u32x4* bv = reinterpret_cast<const u32x4*>(Lw.lora_bv + (size_t)it.g * D * r);
  u32x4* dst = reinterpret_cast<u32x4*>(&sm.vec[0][0]);
  for (int i = threadIdx.x; i < nq16 + nv16; i += kThreads) dst[i] = i < nq16 ? *gl(bq + i) : *gl(bv + i - nq16);
}

// Sum over the 8 lanes of this lane's group (lanes 8 i .. 8 i + 7), in every
// lane of the group; the two halves add in mirrored order, which is exact.
__device__ __forceinline__ float group8_sum(float v) {
  v += DPPF(v, 0xB1, 0xF);   // quad_perm [1,0,3,2]
  v += DPPF(v, 0x4E, 0xF);   // quad_perm [2,3,0,1]
  v += DPPF(v, 0x141, 0xF);  // row_half_mirror
  return v;
}

// Reduce-scatter step over lane bit 5 (d = 32) or 4 (d = 16) with the gfx950
// row swaps: lanes with the bit clear return a + a of the partner lane, lanes
// with it set b + b of the partner.
template <int d>
__device__ __forceinline__ float swap_sum(float a, float b) {
  const auto r = d == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum / sum over the 8 lanes i ^ {0, 8, 16, ..., 56} (lane bits 3..5), in
// every lane; the pairs are combined in mirrored order, so every lane gets
// the same value.
__device__ __forceinline__ float xor_max3(float v) {
  v = fmaxf(v, DPPF(v, 0x128, 0xF));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor_sum3(float v) {
  const float p = DPPF(v, 0x128, 0xF);  // row_ror:8
  v = (threadIdx.x & 8) ? p + v : v + p;
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// This lane's 16 dims of q . k for K fragments kp[0], kp[stride], kp[2 stride],
// kp[3 stride] (16 bytes each: dims 32 k + 4 q8 .. + 3).
__device__ __forceinline__ float dot16(const f32x4 (&q)[4], const u32x4* kp, int stride = 1) {
  float sd = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 kf = as_f4(kp[k * stride]);
    sd = fmaf(q[k].x, kf.x, sd);
    sd = fmaf(q[k].y, kf.y, sd);
    sd = fmaf(q[k].z, kf.z, sd);
    sd = fmaf(q[k].w, kf.w, sd);
  }
  return sd;
}

// Attention item (kv head g, head group, split s), part 1: QK-norm + RoPE of
// the item's q heads and k in LDS, the new cache row, then per head an online
// softmax over the split's positions.  A wave covers 8 positions at a time,
// 8 lanes each: lane q8 of group pg holds dims 32 k + 4 q8 .. + 3 (k < 4) of
// position p_begin + 64 t + 8 wave + pg at step t, so one 8-lane sum gives a
// score.  The 8 group states of a wave are merged in a butterfly and written
// to LDS per head.
template <int G, bool LORA>
__device__ __forceinline__ void attn_phase(const Ctx& c, Smem& sm, int l, const Regs<kFirst>& rg, const AttnPre& pre) {
  const AS4 PersistConst& a = *c.a;
  const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
  const int pos = c.pos, ctx = pos + 1;
  const Item it = item_of<G>(c);
  const int g = it.g, gi = it.gi;
  const int p_begin = it.s * c.chunk, p_end = min(p_begin + c.chunk, ctx);
  const int wave = wave_id(), lane = threadIdx.x & 63, pg = lane >> 3, q8 = lane & 7;
  float* Kg = k_rows(a, l, g);
  float* Vg = v_rows(a, l, g);
  float* qk = sm.qk;
  if (LORA && a.lora_r) {  // q += s B_q u_q on the item's heads, v += s B_v u_v (before QK-norm and RoPE)
    const int r = a.lora_r;
    const uint16_t* bq = reinterpret_cast<const uint16_t*>(&sm.vec[0][0]);
    const uint16_t* bv = bq + gi * D * r;
    const float* u = sm.xres[0];  // u_q, then u_v (polled beside q|k|v)
    for (int row = threadIdx.x; row < (gi + 1) * D; row += kThreads) {
      const bool isq = row < gi * D;
      const uint16_t* b = isq ? bq + row * r : bv + (row - gi * D) * r;
      const float* uu = isq ? u : u + r;
      float t = 0.f;
      for (int k = 0; k < r; ++k) t = fmaf(bf16_to_f(b[k]), uu[k], t);
      qk[isq ? it.j0 * D + row : (G + 1) * D + row - gi * D] += a.lora_scale * t;
    }
    __syncthreads();
  }
  // QK-norm (optional) and RoPE of the item's q heads and k; wave hd handles
  // one of them (lane j: the pair (j, j + 64))
  for (int hd = wave; hd < gi + 1; hd += kWaves) {
    float* v = qk + (hd < gi ? it.j0 + hd : G) * D;
    float x0 = v[lane], x1 = v[lane + 64];
    if (Lw.q_norm) {  // QK-norm present (q and k gains together)
      const float r = rsqrtf(wave_total(x0 * x0 + x1 * x1) / (float)D + a.eps);
      x0 = x0 * r * (hd < gi ? pre.gq0 : pre.gk0);
      x1 = x1 * r * (hd < gi ? pre.gq1 : pre.gk1);
    }
    v[lane] = x0 * pre.ct - x1 * pre.st;
    v[lane + 64] = x1 * pre.ct + x0 * pre.st;
  }
  __syncthreads();
  stamp(c, sm, 5 * l + kAttn, 4, threadIdx.x == 0);
  const float* knew = qk + G * D;
  const float* vnew = qk + (G + 1) * D;
  const float scale = 1.0f / sqrtf((float)D);
  const int pw = p_begin + 8 * wave + pg;  // this lane's position at step 0
  for (int j = 0; j < gi; ++j) {  // the item's heads, one at a time (wave-uniform)
    f32x4 q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = *reinterpret_cast<const f32x4*>(qk + (it.j0 + j) * D + 32 * k + 4 * q8);
    float m = -INFINITY, ls = 0.f;
    f32x4 o[4] = {};
    // steps t0 .. t0 + N/8 - 1 from registers r (K fragments in [0, N/2), V in [N/2, N))
    auto consume = [&](const auto& r, auto n, int t0) {
      constexpr int N = decltype(n)::value, NT = N / 8;
      float sc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sc[t] = -INFINITY;
        const int pf = p_begin + 8 * wave + 64 * (t0 + t);  // the wave's first position of the step
        if (pf >= p_end) continue;  // wave-uniform: no position of the split in this step
        const int p = pw + 64 * (t0 + t);
        float sd = dot16(q, r.R + t * 4);
        if (pf <= pos && pos < pf + 8) {  // wave-uniform: the new position, whose row was loaded before it was written
          const float sn = dot16(q, reinterpret_cast<const u32x4*>(knew + 4 * q8), 8);
          sd = p == pos ? sn : sd;
        }
        sd = group8_sum(sd) * scale;
        sc[t] = p < p_end ? sd : -INFINITY;
      }
      float mx = m;
#pragma unroll
      for (int t = 0; t < NT; ++t) mx = fmaxf(mx, sc[t]);
      if (mx != -INFINITY) {
        const float corr = __expf(m - mx);
        ls *= corr;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = o[k] * corr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int pf = p_begin + 8 * wave + 64 * (t0 + t);
          if (pf >= p_end) continue;  // wave-uniform, as above
          const int p = pw + 64 * (t0 + t);
          const float pwt = __expf(sc[t] - mx);
          ls += pwt;
          if (pf + 8 > p_end || (pf <= pos && pos < pf + 8)) {  // wave-uniform
            // rows past the split were read but are not data (a zero weight
            // times a stale NaN would still be NaN): their V is replaced by 0
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f32x4 vf = p >= p_end ? f32x4{0.f, 0.f, 0.f, 0.f}
                               : p == pos ? *reinterpret_cast<const f32x4*>(vnew + 32 * k + 4 * q8)
                                          : as_f4(r.R[N / 2 + t * 4 + k]);
              o[k] = o[k] + vf * pwt;
            }
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = o[k] + as_f4(r.R[N / 2 + t * 4 + k]) * pwt;
          }
        }
        m = mx;
      }
    };
    consume(rg, std::integral_constant<int, kFirst>{}, 0);
    for (int t0 = kFirst / 8; p_begin + 64 * t0 + 8 * wave < p_end; ++t0) {  // a split longer than the slice loaded ahead
      Addr<kBatch> ad;
      kv_addr<kBatch>(ad, Kg, Vg, p_begin, t0);
      Regs<kBatch> r2;
      load_regs(r2, ad);
      consume(r2, std::integral_constant<int, kBatch>{}, t0);
    }
    if (j == 0) stamp(c, sm, 5 * l + kAttn, 6, threadIdx.x == 0);
    // Merge the 8 groups of the wave (lanes with equal q8 hold the same dims):
    // every group is rescaled to the wave's maximum, then the sums run as a
    // reduce-scatter over lane bits 5 and 4 (each row swap moves two values)
    // and a plain sum over bit 3, leaving o[r] of the wave in lanes 16 r ..
    // 16 r + 15.
    const float M = xor_max3(m);
    const float f = M == -INFINITY ? 0.f : __expf(m - M);
    float ov[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ov[4 * k + 0] = o[k].x * f;
      ov[4 * k + 1] = o[k].y * f;
      ov[4 * k + 2] = o[k].z * f;
      ov[4 * k + 3] = o[k].w * f;
    }
    const float lsum = xor_sum3(ls * f);
    float s8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s8[i] = swap_sum<32>(ov[i], ov[i + 8]);  // bit 5 set: values 8 ..
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] = swap_sum<16>(s8[i], s8[i + 4]);  // bit 4 set: values 4 ..
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[i] += DPPF(s4[i], 0x128, 0xF);  // row_ror:8: lanes i, i ^ 8
    if ((lane & 8) == 0) {  // the wave's state of head j: o[r] from row r's lanes 0..7
      float* e = sm.att + (wave * G + j) * kAttStride;
      *reinterpret_cast<f32x4*>(e + 4 + 32 * (lane >> 4) + 4 * q8) = f32x4{s4[0], s4[1], s4[2], s4[3]};
      if (lane == 0) {
        e[0] = M;
        e[1] = lsum;
      }
    }
  }
}

// Attention item, part 2: combine the 8 wave states in a fixed order into this
// split's partial (with one split, into the output); then the item's heads j
// with j % S == s fold the S split partials in split order.
template <int G>
__device__ __forceinline__ bool attn_finish(const Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const Item it = item_of<G>(c);
  const int S = c.S, s = it.s, gi = it.gi, h0 = it.g * G + it.j0;  // h0: the item's first q head
  const uint32_t tag = tag_of(c.seq, l);
  __syncthreads();
  stamp(c, sm, 5 * l + kAttn, 7, threadIdx.x == 0);
  for (int idx = threadIdx.x; idx < gi * D; idx += kThreads) {
    const int j = idx / D, dd = idx % D;
    float mw[kWaves], lw[kWaves], ow[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* e = sm.att + (w * G + j) * kAttStride;
      mw[w] = e[0];
      lw[w] = e[1];
      ow[w] = e[4 + dd];
    }
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, mw[w]);
    float Ls = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {  // a wave without positions has m = -inf: weight 0
      const float f = __expf(mw[w] - M);
      Ls += lw[w] * f;
      acc += ow[w] * f;
    }
    const int h = h0 + j;
    if (S == 1) {  // value pairs: the even lane stores its own and its neighbour's (dd ^ 1) value
      const float v = acc / Ls;
      const float vn = DPPF(v, 0xB1, 0xF);
      if ((dd & 1) == 0) st_pair(a.O + ((h * D + dd) >> 1), v, vn, tag);
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
  const int nmerge = s < gi ? (gi - 1 - s) / S + 1 : 0;
  bool ok = true;
  for (int t0 = 0; t0 < nmerge * D; t0 += kThreads) {
    const int t = t0 + threadIdx.x;
    const bool act = t < nmerge * D;
    const int j = s + (t / D) * S, dd = t % D;
    const int h = h0 + (act ? j : 0);
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
    const float v = acc / Ls;
    const float vn = DPPF(v, 0xB1, 0xF);  // dims dd, dd ^ 1 sit in neighbouring lanes
    if (ok && act && (dd & 1) == 0) st_pair(a.O + ((h * D + dd) >> 1), v, vn, tag);
  }
  if (!ok) sm.abort_flag = 1;
  __syncthreads();
  return !sm.abort_flag;
}

// Attention item, part 3: the new position's K/V row into the cache, by the
// item whose split holds it.  Only later steps read the row (this step uses
// the LDS copy), so it is written after the outputs: a store still in flight
// would make the memory waits of the combine wait for it.
template <int G>
__device__ __forceinline__ void attn_cache_write(const Ctx& c, Smem& sm, int l) {
  const AS4 PersistConst& a = *c.a;
  const Item it = item_of<G>(c);
  const int pos = c.pos, p_begin = it.s * c.chunk, p_end = min(p_begin + c.chunk, pos + 1);
  if (it.x == 0 && pos >= p_begin && pos < p_end && threadIdx.x < D) {
    st_f(k_rows(a, l, it.g) + (size_t)pos * D + threadIdx.x, sm.qk[G * D + threadIdx.x]);
    st_f(v_rows(a, l, it.g) + (size_t)pos * D + threadIdx.x, sm.qk[(G + 1) * D + threadIdx.x]);
  }
}

// LM head: rows wave, wave + 8, ... of this CU's vocabulary slice, logits
// out, per-CU argmax (ties -> lowest id) as a tagged pair.  The registers
// loaded ahead hold three batches of kBatch segments (kBatch / HS rows per
// wave each); each batch, once consumed, is reloaded with the rows three
// batches on, so two batches stream while one is consumed.
template <int HS>
__device__ __forceinline__ void lmhead_phase(const Ctx& c, Smem& sm, Regs<kFirst>& rg, float rs) {
  static_assert(kFirst == 3 * kBatch, "three streamed batches");
  const AS4 PersistConst& a = *c.a;
  const int v0 = c.v0, nrows = c.v1 - c.v0, lane = threadIdx.x & 63, wave = wave_id();
  const float* h = sm.vec[a.L & 1];
  const __amdgpu_buffer_rsrc_t E = rsrc_of(a.embed + (size_t)v0 * HS * kSeg);  // this CU's first row
  constexpr int RB = kBatch / HS;        // rows of a wave in one batch
  constexpr int step = RB * kWaves;      // rows of one batch (all waves)
  float best = -INFINITY;
  int bi = 0x7fffffff;
  auto run = [&](auto j, int rb) {  // batch j of the three: rows rb, rb + 8, ...
    constexpr int o = decltype(j)::value * kBatch;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int rr = rb + i * kWaves;
      if (rr < nrows) {  // wave-uniform
        float acc = 0.f;
#pragma unroll
        for (int sg = 0; sg < HS; ++sg) acc += dot8(rg.R[o + i * HS + sg], h + sg * kSeg + lane * 8);
        const float t = wave_total(acc) * rs;
        if (lane == 0) sm.outv[rr] = t;
        if (t > best) {  // a wave's rows increase: ties keep the lowest id
          best = t;
          bi = v0 + rr;
        }
      }
    }
    const int rn = rb + 3 * step;
    if (rn < nrows) {  // wave-uniform: reload this batch with the rows three batches on
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int rr = min(rn + i * kWaves, nrows - 1);
#pragma unroll
        for (int sg = 0; sg < HS; ++sg)
          rg.R[o + i * HS + sg] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(E, lane * 16, (rr * HS + sg) * kSeg * 2, 2 /* nt */));
      }
    }
  };
  for (int rb = wave; rb < nrows; rb += 3 * step) {
    run(std::integral_constant<int, 0>{}, rb);
    run(std::integral_constant<int, 1>{}, rb + step);
    run(std::integral_constant<int, 2>{}, rb + 2 * step);
  }
  if (lane == 0) {
    sm.red[32 + wave] = best;
    sm.red[40 + wave] = __int_as_float(bi);
  }
  __syncthreads();
  for (int rr = threadIdx.x; rr < nrows; rr += kThreads) st_f(a.logits + v0 + rr, sm.outv[rr]);
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
__device__ __forceinline__ void final_phase(const Ctx& c, Smem& sm, int k, int32_t* tokens_out) {
  const AS4 PersistConst& a = *c.a;
  const int n = gridDim.x, ph = 5 * a.L + 1, slot = a.L + 1;  // the LM head used slot L
  float* vals = sm.vec[slot & 1];
  float rs;
  stamp(c, sm, ph, 0, threadIdx.x == 0);
  if (!poll(c, sm, slot, a.AM, 2 * n, tag_of(c.seq, 255), vals, nullptr, &rs, nullptr, 0, nullptr)) return;
  stamp(c, sm, ph, 1, threadIdx.x == 0);
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
    if (tokens_out) *gl(tokens_out + k) = j;
    // the token for the launch's next step, after the step state
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(gl(a.TOK), ((uint64_t)tag_of(c.seq, kTokLayer) << 32) | (uint32_t)j, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  stamp(c, sm, ph, 5, lane == 0);
}

// Gate before a poll: lane 0 of wave 0 watches one word of the producer's own
// input, sleeping between reads, while the other waves wait at the barrier;
// once it carries tag `gtag` (or a later one) the producer is at work and the
// full poll starts, so the input vector is not polled at full rate through
// the whole wait.  Returns false when the step is abandoned.
__device__ __forceinline__ bool gate(const Ctx& c, Smem& sm, const uint64_t* w, uint32_t gtag, bool packed = false) {
  if (threadIdx.x == 0) {
    uint32_t spin = 0;
    auto early = [&](uint64_t v) {  // tag before gtag (packed words: 16-bit tags)
      return packed ? (int16_t)(uint16_t)((uint32_t)(v >> 48) - gtag) < 0 : (int32_t)((uint32_t)(v >> 32) - gtag) < 0;
    };
    while (early(ld_tagged(w))) {
      if ((++spin & 3) == 0 && timed_out(c)) {
        st_u32(&c.a->err[0], 1);
        sm.abort_flag = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(32);
    }
  }
  lds_barrier();
  return !sm.abort_flag;
}

template <int G, int HS, bool Q4, bool LORA>
__global__ __launch_bounds__(kThreads, 1) void k_decode_persistent(const PersistConst* __restrict__ pc,
                                                                   PersistStep stp) {
  extern __shared__ __align__(16) char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  if (threadIdx.x == 0) sm.abort_flag = 0;
  if (pc->trace)
    for (int i = threadIdx.x; i < (kTraceL + 2) * 8; i += kThreads) sm.ts[i / 8][i % 8] = 0;
  const AS4 PersistConst* ap = (const AS4 PersistConst*)pc;
  const AS4 PersistConst& a = *ap;
  Ctx c;
  c.a = ap;
  c.pos = stp.pos;
  c.S = stp.S;
  c.chunk = stp.chunk;
  c.X = stp.X;
  c.eps = a.eps;
  c.seq = stp.seq;
  c.t0 = __builtin_amdgcn_s_memrealtime();
  int role = 0;
  while (role < 4 && (int)blockIdx.x >= stp.start[role + 1]) ++role;
  c.role = role;
  c.rank = (int)blockIdx.x - stp.start[role];
  c.nrole = stp.start[role + 1] - stp.start[role];
  const int N = role == kQKV ? a.nqkv : role == kGateUp ? a.I : role == kAttn ? c.nrole : a.H;
  // with an adapter the QKV role's last CU computes the LoRA down products
  const int nr = c.nrole - (LORA && role == kQKV && a.lora_r > 0 ? 1 : 0);
  const bool lora = LORA && c.rank >= nr;
  if (lora) {
    c.r0 = a.nqkv;
    c.r1 = a.nqkv + 2 * a.lora_r;
  } else if (role != kAttn && N % 16 == 0 && N / 16 >= nr) {  // whole 16-row tile blocks (no overlapping block)
    c.r0 = 16 * (int)(((uint32_t)(N / 16) * c.rank) / nr);
    c.r1 = 16 * (int)(((uint32_t)(N / 16) * (c.rank + 1)) / nr);
  } else if (role == kGateUp) {  // even boundaries: the activations travel as value pairs
    c.r0 = 2 * (int)(((uint32_t)(N / 2) * c.rank) / nr);
    c.r1 = 2 * (int)(((uint32_t)(N / 2) * (c.rank + 1)) / nr);
  } else {
    c.r0 = (int)(((uint32_t)N * c.rank) / nr);
    c.r1 = (int)(((uint32_t)N * (c.rank + 1)) / nr);
  }
  c.v0 = (int)(((uint32_t)a.V * blockIdx.x) / gridDim.x);
  c.v1 = (int)(((uint32_t)a.V * (blockIdx.x + 1)) / gridDim.x);
  const int L = a.L, H = a.H, tid = threadIdx.x;
  Regs<kFirst> rg;
  for (int k = 0; k < stp.nsteps; ++k) {  // decode steps of this launch, each one's token feeding the next
  int token;
  if (k == 0) {
    token = gl(a.st)->token;
  } else {
    // the next position: the same splits, each one position longer (as the
    // per-step plan would cut them), and the token the last step chose
    c.pos = stp.pos + k;
    c.seq = stp.seq + k;
    c.t0 = __builtin_amdgcn_s_memrealtime();
    c.chunk = step_chunk(c.pos + 1, (int)gridDim.x, a.nkv);
    if (tid == 0) {
      const uint64_t want = (uint64_t)tag_of(c.seq - 1, kTokLayer) << 32;
      uint64_t v;
      uint32_t spin = 0;
      while (((v = ld_tagged(a.TOK)) >> 32) != (want >> 32)) {
        if ((++spin & 31) == 0 && timed_out(c)) {
          st_u32(&c.a->err[0], 1);
          sm.abort_flag = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      sm.red[47] = __int_as_float((int)(uint32_t)v);
    }
    __syncthreads();
    if (sm.abort_flag) return;
    token = __float_as_int(sm.red[47]);
    // every row the last step wrote (the K/V cache rows) is read afresh
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  const uint16_t* emb = a.embed + (size_t)token * H;
  load_regs(rg, ahead_addr<HS, Q4, LORA>(c, 0, lora));
  __syncthreads();
  for (int l = 0; l < L; ++l) {
    const int ph = 5 * l + role;
    const AS4 LayerPtrs& Lw = ((const AS4 LayerPtrs*)a.layers)[l];
    const uint32_t tag = tag_of(c.seq, l);
    float* vin = sm.vec[l & 1];
    float* xr = sm.xres[l & 1];
    float rs = 1.0f;
    stamp(c, sm, ph, 0, tid == 0);
    // everything the phase needs that does not depend on its input is read
    // before the input poll, so its latency hides behind the handshake
    AttnPre pre{};
    Gemv gv{};
    const float* bias = nullptr;
    if (role == kAttn) {
      pre = attn_pre(c, l);
      if (LORA && a.lora_r) lora_stage<G>(c, sm, l);
    } else if (!lora) {
      if (!Q4) gv = gemv_of(c, l);
      if (role == kQKV) bias = Lw.bqkv;
    }
    // ---- the phase input and the compute
    Tiles tw;
    if (!Q4 && role != kAttn && !lora && !(l == 0 && role == kQKV) && mfma_path(c, &tw)) {
      if (!gemv_waves(c, sm, l, rg, tw, bias)) return;  // per-wave input, matrix-core rows
    } else {
      bool ok = true;
      // int4 roles: the group scales of the slots loaded ahead, requested
      // before the input wait (1/64 of the codes' bytes)
      uint32_t sc[kFirst];
      if (Q4 && role != kAttn && !lora) {
        SAddr<kFirst> sa;
        q4_saddr<kFirst>(sa, q4_geo(c, l), 0);
        load_scales<0>(sc, sa);
      }
      {  // the word the gate watches: the producer's input (f32 vectors only)
        const uint64_t* gw = nullptr;
        uint32_t gt = tag;
        switch (role) {
          case kQKV: if (l > 0) { gw = a.X1; gt = tag_of(c.seq, l - 1); } break;
          case kAttn: if (l > 0) gw = a.X0; break;
          case kOproj: gw = a.QKV; break;
          case kGateUp: gw = a.O; break;  // value pairs
          default: gw = a.X1; break;
        }
        if (gw && !gate(c, sm, gw, gt, role == kGateUp)) return;
      }
      if (l == 0 && role == kQKV) {  // layer 0: x0 is the embedding row (nothing to wait for)
        float ss = 0.f;
        const bool split = !Q4 && !lora && mfma_path(c);
        for (int k = tid; k < H; k += kThreads) {
          const float x = bf16_to_f(*gl(emb + k));
          const float y = x * ld_f(Lw.attn_norm + k);
          if (split) {
            uint16_t* d = reinterpret_cast<uint16_t*>(vin) + (k >> 3) * 16 + (k & 7);
            const uint32_t hb = bf16_rne(y);
            d[0] = (uint16_t)hb;
            d[8] = (uint16_t)bf16_rne(y - __uint_as_float(hb << 16));
          } else {
            vin[k] = y;
          }
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
        switch (role) {
          case kQKV: src = a.X0; n = H; gain = Lw.attn_norm; break;
          case kAttn:
            src = a.QKV + (size_t)(c.rank / (c.X * c.S)) * (G + 2) * D;
            n = (G + 2) * D;
            dst = sm.qk;
            if (LORA && a.lora_r) {  // the LoRA down products u_q, u_v
              src2 = a.QKV + a.nqkv;
              n2 = 2 * a.lora_r;
              xr = sm.xres[0];
            }
            break;
          case kOproj:
            src = a.O;
            n = a.nq * D;
            if (l == 0) {
              for (int r = tid; r < c.r1 - c.r0; r += kThreads) xr[r] = bf16_to_f(*gl(emb + c.r0 + r));
            } else {
              src2 = a.X0 + c.r0;
              n2 = c.r1 - c.r0;
            }
            break;
          case kGateUp: src = a.X1; n = H; gain = Lw.mlp_norm; break;
          default: src = a.ACT; n = a.I; src2 = a.X1 + c.r0; n2 = c.r1 - c.r0; break;
        }
        // (int4 roles hold their slots' scales meanwhile: a narrower poll keeps
        // the registers within one wave per SIMD half)
        ok = poll<Q4 ? 4 : kPE>(c, sm, l, src, n, tag, dst, gain, &rs, src2, n2, xr, role == kOproj || role == kDown);
      }
      if (!ok) return;
      stamp(c, sm, ph, 1, tid == 0);
      // ---- compute from the registers loaded a layer ahead
      if (role == kAttn) {
        attn_phase<G, LORA>(c, sm, l, rg, pre);
        stamp(c, sm, ph, 2, tid == 0);
        if (!attn_finish<G>(c, sm, l)) return;
        attn_cache_write<G>(c, sm, l);
        if (stp.nsteps > 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // the row before later steps read it
      } else if (LORA && lora) {
        lora_phase(c, sm, l, rg, rs);
      } else {
        gemv_phase<Q4>(c, sm, l, rg, sc, rs, gv, bias);
      }
    }
    stamp(c, sm, ph, 3, tid == 0);
    // the single load site: the next layer's slice (after the last layer, the
    // first LM-head rows) streams while the other roles take their phases
    load_regs(rg, ahead_addr<HS, Q4, LORA>(c, l + 1, lora));
    stamp(c, sm, ph, 5, tid == 0);
  }
  // ---- final norm + LM head (every CU)
  {
    const int ph = 5 * L;
    float rs;
    stamp(c, sm, ph, 0, tid == 0);
    if (!gate(c, sm, a.X1, tag_of(c.seq, L - 1))) return;
    if (!poll(c, sm, L, a.X0, H, tag_of(c.seq, L), sm.vec[L & 1], a.final_norm, &rs, nullptr, 0, nullptr)) return;
    stamp(c, sm, ph, 1, tid == 0);
    if (blockIdx.x == 0 && a.xf_out)
      for (int k = tid; k < H; k += kThreads) st_f(a.xf_out + k, sm.vec[L & 1][k] * rs);
    lmhead_phase<HS>(c, sm, rg, rs);
    stamp(c, sm, ph, 5, tid == 0);
  }
  if (blockIdx.x == 0) final_phase(c, sm, k, stp.tokens_out);
  if (sm.abort_flag) return;
  }  // decode steps
  if (a.trace) {
    __syncthreads();
    trace_flush(c, sm);
  }
}

template <int G, int HS, bool Q4, bool LORA>
void* kernel_ptr() {
  return (void*)k_decode_persistent<G, HS, Q4, LORA>;
}

template <bool Q4, bool LORA>
void* pick_fmt(int G, int hseg) {
  if (hseg == 2) {
    switch (G) {
      case 1: return kernel_ptr<1, 2, Q4, LORA>();
      case 2: return kernel_ptr<2, 2, Q4, LORA>();
      case 4: return kernel_ptr<4, 2, Q4, LORA>();
      case 8: return kernel_ptr<8, 2, Q4, LORA>();
    }
  } else if (hseg == 4) {
    switch (G) {
      case 1: return kernel_ptr<1, 4, Q4, LORA>();
      case 2: return kernel_ptr<2, 4, Q4, LORA>();
      case 4: return kernel_ptr<4, 4, Q4, LORA>();
      case 8: return kernel_ptr<8, 4, Q4, LORA>();
    }
  }
  return nullptr;
}

// The kernels with the LoRA-down CU and the attention items' up products are
// separate instantiations, so that the adapter's code takes no registers from
// the kernels without one.
void* pick(int G, int hseg, int q4, int lora) {
  if (lora) return q4 ? pick_fmt<true, true>(G, hseg) : pick_fmt<false, true>(G, hseg);
  return q4 ? pick_fmt<true, false>(G, hseg) : pick_fmt<false, false>(G, hseg);
}

// Segments one wave of a CU with `units` units (rpu rows of nseg segments) loads.
int wave_segs(int units, int rpu, int nseg) { return (units + kWaves - 1) / kWaves * rpu * nseg; }

}  // namespace

size_t persist_smem_bytes() { return sizeof(Smem); }

int persist_prepare(int G, int hseg, int q4, int lora) {
  void* fn = pick(G, hseg, q4, lora);
  if (!fn) return -1;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
  if (e != hipSuccess) return (int)e;
  int per_cu = 0;  // one workgroup per CU must fit (the grid is one per CU)
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, sizeof(Smem));
  if (e != hipSuccess) return (int)e;
  return per_cu >= 1 ? 0 : -1;
}

int persist_plan(const PersistConst& pc, int grid, int pos, uint32_t seq, PersistStep* out) {
  if (grid < 1 || pos < 0 || pos >= pc.max_pos || pc.nkv < 1) return -1;
  if (pc.I % 2 != 0) return -1;  // the SwiGLU activations travel as value pairs
  const int ctx = pos + 1;
  // attention: splits no longer than the K/V rows a CU loads ahead, on at most half the grid
  if (grid / (2 * pc.nkv) < 1) return -1;
  int chunk;
  const int S = split_plan(ctx, grid, pc.nkv, &chunk);
  // short contexts: one item per q head (X = G head groups) instead of one per
  // kv head, which halves (or better) the serial work of an item; each group
  // reads the kv head's rows again, which is cheap while they are few
  const int G = pc.nq / pc.nkv;
  const int X = (S == 1 && pc.nkv * G <= grid / 4) ? G : 1;
  const int nl = pc.lora_r > 0 ? 1 : 0;  // the LoRA-down CU (last of the QKV role)
  const int R = grid - pc.nkv * X * S - nl;
  if (pc.q4) {  // int4 roles: whole 16-row blocks, CUs in proportion to the slots (16 rows x 128 columns)
    const int NB[4] = {pc.nqkv / 16, pc.H / 16, pc.I / 16, pc.H / 16};
    const int NG[4] = {pc.H / 128, pc.nq * D / 128, pc.H / 128, pc.I / 128};
    const int sets[4] = {1, 1, 2, 1};
    const int att_rows = (int)(sizeof(Smem::att) / sizeof(float)) / kWaves;  // LDS partial rows of a CU
    int n[4], lo_sum = 0;
    for (int r = 0; r < 4; ++r) {
      int lo = 1;
      if (r == 1 || r == 3) lo = std::max(lo, (pc.H + kResMax - 1) / kResMax);  // residual rows fit the LDS slot
      while ((NB[r] + lo - 1) / lo * 16 * sets[r] > att_rows) ++lo;
      if (lo > NB[r]) return -1;
      n[r] = lo;
      lo_sum += lo;
    }
    if (lo_sum > R) return -1;
    // the phases run one after another, so the spare CUs go where they cut
    // the most slots per wave (the busiest wave of a CU: ceil(NB / n) blocks
    // per row set, ceil(NG / 8) groups each), slots beyond the registers
    // loaded ahead (which stream in during the phase, their load latency
    // exposed) counted seven times; whole steps only, as a block count per CU
    // drops at certain n
    auto cost = [&](int r, int m) {
      const int spw = sets[r] * ((NB[r] + m - 1) / m) * ((NG[r] + kWaves - 1) / kWaves);
      return spw + 6 * std::max(0, spw - kFirst);
    };
    int left = R - lo_sum;
    while (left > 0) {
      int best = -1, bk = 0;
      double bg = 0.0;
      for (int r = 0; r < 4; ++r) {
        const int c0 = cost(r, n[r]);
        for (int k = 1; k <= left && n[r] + k <= NB[r]; ++k) {
          const int c1 = cost(r, n[r] + k);
          if (c1 < c0) {
            const double g = (double)(c0 - c1) / k;
            if (g > bg) {
              bg = g;
              best = r;
              bk = k;
            }
            break;
          }
        }
      }
      if (best < 0) {  // no step left that helps: the rest to the busiest role that can take them
        int r1 = -1;
        for (int r = 0; r < 4; ++r)
          if (n[r] < NB[r] && (r1 < 0 || cost(r, n[r]) > cost(r1, n[r1]))) r1 = r;
        if (r1 < 0) break;
        best = r1;
        bk = 1;
      }
      n[best] += bk;
      left -= bk;
    }
    out->nsteps = 1;
    out->tokens_out = nullptr;
    out->pos = pos;
    out->seq = seq;
    out->S = S;
    out->chunk = chunk;
    out->X = X;
    out->start[0] = 0;
    out->start[1] = n[0] + nl;
    out->start[2] = out->start[1] + pc.nkv * X * S;
    out->start[3] = out->start[2] + n[1];
    out->start[4] = out->start[3] + n[2];
    out->start[5] = out->start[4] + n[3];
    return out->start[5] == grid ? 0 : -1;
  }
  // the GEMV roles: Q rows, O rows, gate/up row pairs, D rows
  const int N[4] = {pc.nqkv, pc.H, pc.I, pc.H};
  const int rpu[4] = {1, 1, 2, 1};
  const int ns[4] = {(pc.H + kSeg - 1) / kSeg, (pc.nq * D + kSeg - 1) / kSeg, (pc.H + kSeg - 1) / kSeg,
                     (pc.I + kSeg - 1) / kSeg};
  int lo[4];
  for (int r = 0; r < 4; ++r) lo[r] = 1;
  lo[1] = (pc.H + kResMax - 1) / kResMax;  // residual rows of a CU fit its LDS slot
  lo[3] = lo[1];
  for (int r = 0; r < 4; ++r) lo[r] = std::max(lo[r], (N[r] + kOutMax - 1) / kOutMax);  // outputs fit too
  if ((pc.V + grid - 1) / grid > kOutMax) return -1;
  // gate/up publishes value pairs: every CU of it owns at least one pair
  const int cap[4] = {N[0], N[1], N[2] / 2, N[3]};
  int lo_sum = 0, tmax = 0;
  for (int r = 0; r < 4; ++r) {
    if (cap[r] < lo[r]) return -1;
    lo_sum += lo[r];
    tmax = std::max(tmax, wave_segs((N[r] + lo[r] - 1) / lo[r], rpu[r], ns[r]));
  }
  if (lo_sum > R) return -1;
  // the smallest per-wave slice every role can meet with R CUs, then the
  // spare CUs to the roles with the most segments per CU
  int n[4] = {lo[0], lo[1], lo[2], lo[3]};
  for (int T = 1; T <= tmax; ++T) {
    int m[4], sum = 0;
    bool fits = true;
    for (int r = 0; r < 4 && fits; ++r) {
      const int per = T / (rpu[r] * ns[r]);  // units per wave
      if (per == 0) {
        fits = false;
        break;
      }
      m[r] = std::min(cap[r], std::max(lo[r], (N[r] + kWaves * per - 1) / (kWaves * per)));
      sum += m[r];
    }
    if (fits && sum <= R) {
      for (int r = 0; r < 4; ++r) n[r] = m[r];
      break;
    }
  }
  for (int sum = n[0] + n[1] + n[2] + n[3]; sum < R; ++sum) {
    int best = -1;
    double bw = -1.0;
    for (int r = 0; r < 4; ++r) {
      if (n[r] >= cap[r]) continue;
      const double w = (double)N[r] * rpu[r] * ns[r] / n[r];
      if (w > bw) {
        bw = w;
        best = r;
      }
    }
    if (best < 0) break;
    ++n[best];
  }
  out->nsteps = 1;
  out->tokens_out = nullptr;
  out->pos = pos;
  out->seq = seq;
  out->S = S;
  out->chunk = chunk;
  out->X = X;
  out->start[0] = 0;
  out->start[1] = n[0] + nl;
  out->start[2] = out->start[1] + pc.nkv * X * S;
  out->start[3] = out->start[2] + n[1];
  out->start[4] = out->start[3] + n[2];
  out->start[5] = out->start[4] + n[3];
  return out->start[5] == grid ? 0 : -1;  // every CU has a role
}

// The step needs all grid workgroups resident at once (one per CU).  A plain
// launch gets that on a device that runs nothing else: the previous work on
// the stream has completed and every CU takes one workgroup.  A cooperative
// launch would guarantee it, but costs ~19 us more per step here.  If the
// device is shared and a workgroup cannot start, the resident ones give up
// after their bounded wait and the step is reported as abandoned.
int persist_batch_len(const PersistConst& pc, int grid, int pos, int nmax) {
  int ch;
  const int S = split_plan(pos + 1, grid, pc.nkv, &ch);
  int m = 1;
  while (m < nmax && pos + m < pc.max_pos && split_plan(pos + m + 1, grid, pc.nkv, &ch) == S) ++m;
  return m;
}

int persist_launch(const PersistConst* dev_const, int G, int hseg, int q4, int lora, int grid,
                   const PersistStep& st, hipStream_t s) {
  void* fn = pick(G, hseg, q4, lora);
  if (!fn) return -1;
  PersistStep arg = st;
  void* args[] = {(void*)&dev_const, (void*)&arg};
  hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, sizeof(Smem), s);
  return e == hipSuccess ? 0 : (int)e;
}
