// Split-K flash-decode attention for one new row (the decode step), GQA.
//
// "EMBERGLASS (qwen-webgpu-lora) README", split-K decode attention: the cache
// positions 0 .. ctx-1 are cut into S splits; each split produces the
// unnormalised softmax state {max m, sum l, weighted values o} of its
// positions, and a merge combines the splits.  Here a block of 256 threads
// owns one kv head g and one split, and handles the G = nq / nkv query heads
// of g together, so each K/V row is read from HBM once for the whole group.
//
// The split count S is fixed for the life of the engine (so one captured
// graph serves every position); the split length is C = max(cmin, ceil(ctx /
// S)), computed on the device from the step state, and splits past the end of
// the context do nothing.
//
// The block also finishes the new row's q and k: the raw q|k|v projection of
// its group is read, q and k get the per-head RMSNorm (when the model has it)
// and RoPE at the new position ("flashmoon demo/README.md", RoPE applied as K
// is written), and the block whose split ends at the new position writes k
// and v into the cache for later steps and uses them from LDS for this one.
// Within a split, positions go in tiles of 64:
//   1. each thread loads 32 dims of K and of V of one position (4 threads per
//      position, 16-byte loads, a wave reads 16 consecutive rows);
//   2. scores s = q_j . k / sqrt(d) from K in registers and q in LDS;
//   3. per head, the running max / sum are updated (online softmax) and the
//      tile's probabilities written to LDS;
//   4. each thread rescales and accumulates its (head, dim) outputs from the V
//      tile in LDS.
// Every sum has a fixed order, so results are identical run to run.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int D = 128;
constexpr int TP = 64;  // positions per tile

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  const float t = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return t;
}

__device__ __forceinline__ int split_len(int ctx, int S, int cmin) { return max(cmin, (ctx + S - 1) / S); }

// grid (nkv, S), block 256.  Partials part[h][s] = {m, l, o[0..D)} for query
// head h = g G + j (o not divided by l).
// One head of the new row: optional RMSNorm over its D values (gain), then
// RoPE with the half-split pairing (j, j + D/2) at table row `pos`.  Lane l of
// the wave holds dims l and l + 64; the results go to out[l], out[l + 64].
__device__ __forceinline__ void norm_rope_head(const float* __restrict__ src, const float* __restrict__ gain,
                                               float eps, const float* __restrict__ cos_t,
                                               const float* __restrict__ sin_t, int pos, float* out) {
  const int l = threadIdx.x & 63;
  float a = src[l], b = src[l + 64];
  if (gain) {
    const float r = 1.0f / sqrtf(wave_sum(a * a + b * b) / (float)D + eps);
    a = a * r * gain[l];
    b = b * r * gain[l + 64];
  }
  const float c = cos_t[(size_t)pos * (D / 2) + l], s = sin_t[(size_t)pos * (D / 2) + l];
  out[l] = a * c - b * s;
  out[l + 64] = b * c + a * s;
}

// With an adapter (LORA), the block first adds the up products of its heads:
// q_j += s B_q u_q and v += s B_v u_v ("EMBERGLASS (qwen-webgpu-lora) README",
// LoRA sections), u = [A_q; A_v] h from the down-product GEMV, before QK-norm
// and RoPE; one thread per adapted row.
struct LoraUp {
  const float* u;      // [2 r]: u_q, u_v
  const uint16_t* bq;  // [nq d][r] bf16
  const uint16_t* bv;  // [nkv d][r] bf16
  int r;
  float scale;
};

template <int G, bool LORA, typename KVT>
__global__ __launch_bounds__(256) void k_attn_decode(const float* __restrict__ qkv, const float* __restrict__ qn,
                                                     const float* __restrict__ kn, float eps,
                                                     const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                                                     KVT* __restrict__ Kc, KVT* __restrict__ Vc, int max_pos,
                                                     const DevState* __restrict__ st, int row, int S, int cmin, float scale,
                                                     float* __restrict__ part, LoraUp lu) {
  const int g = blockIdx.x, sp = blockIdx.y;
  const int ctx = st->pos + row + 1, pos = ctx - 1;  // (row: of a batch of new rows)
  const int C = split_len(ctx, S, cmin);
  const int p_begin = sp * C;
  if (p_begin >= ctx) return;  // the merge reads only the splits that hold positions
  const int p_end = min(p_begin + C, ctx);

  __shared__ __align__(16) float qs[G * D];
  __shared__ __align__(16) float vs[TP * D];
  __shared__ __align__(16) float ps[G * TP];  // scores, then probabilities
  __shared__ float cs[G];                     // per-head rescale of this tile
  __shared__ __align__(16) float kv_new[2 * D];  // k (normed, rotated) and v of the new row

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // group-major projection rows: [q heads g G .. g G + G - 1 | k_g | v_g] x D
  const float* grp = qkv + (size_t)g * (G + 2) * D;
  const float* qsrc = grp;          // the q heads' raw rows
  const float* vsrc = grp + (G + 1) * D;  // and v's
  if (LORA) {  // q and v with the adapter, into the V tile's LDS (free until the first tile)
    float* raw = vs;  // [G D | D]
    float* us = vs + (G + 1) * D;  // u_q | u_v, after them
    const int r = lu.r;
    if (tid < 2 * r) us[tid] = lu.u[tid];
    __syncthreads();
    for (int row = tid; row < (G + 1) * D; row += 256) {
      const bool isq = row < G * D;
      const uint16_t* b = isq ? lu.bq + ((size_t)g * G * D + row) * r : lu.bv + ((size_t)g * D + row - G * D) * r;
      const float* u = us + (isq ? 0 : r);
      float a = 0.f;  // (rows of B are r values apart, any r)
      for (int k = 0; k < r; ++k) a = fmaf(bf16_to_f(b[k]), u[k], a);
      raw[row] = (isq ? grp[row] : grp[(G + 1) * D + row - G * D]) + lu.scale * a;
    }
    __syncthreads();
    qsrc = raw;
    vsrc = raw + G * D;
  }
  for (int j = wave; j < G; j += 4) norm_rope_head(qsrc + j * D, qn, eps, cos_t, sin_t, pos, qs + j * D);
  const bool owns_new = p_end == ctx;
  if (owns_new && wave == 3) {  // wave 3 has the fewest q heads
    norm_rope_head(grp + G * D, kn, eps, cos_t, sin_t, pos, kv_new);
    // the new row as the cache stores it (bf16 cache: rounded), for this step too
    const float k0 = kv_round<KVT>(kv_new[lane]), k1 = kv_round<KVT>(kv_new[lane + 64]);
    const float v0 = kv_round<KVT>(vsrc[lane]), v1 = kv_round<KVT>(vsrc[64 + lane]);
    kv_new[lane] = k0;
    kv_new[lane + 64] = k1;
    kv_new[D + lane] = v0;
    kv_new[D + 64 + lane] = v1;
    KVT* kr = Kc + ((size_t)g * max_pos + pos) * D;
    KVT* vr = Vc + ((size_t)g * max_pos + pos) * D;
    st_kv(kr + lane, k0);
    st_kv(kr + lane + 64, k1);
    st_kv(vr + lane, v0);
    st_kv(vr + lane + 64, v1);
  }

  const int pl = tid >> 2, sub = tid & 3;  // load / score mapping: position, quarter of the dims
  // output mapping: G < 8: dim dd of heads jh, jh + 2, ...; G = 8: dims
  // 4 dq .. + 3 of head hq (one 16-byte V read feeds four products)
  const int dd = tid & 127, jh = tid >> 7;
  const int dq = tid & 31, hq = tid >> 5;
  constexpr bool QUAD = G == 8;
  constexpr int JPT = QUAD ? 1 : (G >= 2 ? G / 2 : 1);  // output heads per thread
  constexpr int HPW = G >= 4 ? G / 4 : 1;  // softmax heads per wave
  float acc[JPT];
#pragma unroll
  for (int i = 0; i < JPT; ++i) acc[i] = 0.f;
  f32x4 acc4 = f32x4{0.f, 0.f, 0.f, 0.f};
  float M[HPW], L[HPW];
#pragma unroll
  for (int r = 0; r < HPW; ++r) { M[r] = -INFINITY; L[r] = 0.f; }

  const KVT* Kg = Kc + (size_t)g * max_pos * D;
  const KVT* Vg = Vc + (size_t)g * max_pos * D;
  for (int t0 = p_begin; t0 < p_end; t0 += TP) {
    const int n = min(TP, p_end - t0);
    f32x4 kr[8], vr[8];
    const bool fresh = owns_new && t0 + pl == pos;  // the new row: from LDS, not the cache
    if (pl < n && !fresh) {
      const size_t off = (size_t)(t0 + pl) * D + sub * 32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kr[i] = ld_kv4(Kg + off + 4 * i);
        vr[i] = ld_kv4(Vg + off + 4 * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();  // q (and the new k, v) staged; the previous tile's V and probabilities consumed
    if (fresh) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kr[i] = reinterpret_cast<const f32x4*>(kv_new + sub * 32)[i];
        vr[i] = reinterpret_cast<const f32x4*>(kv_new + D + sub * 32)[i];
      }
    }
    if (pl < n) {
#pragma unroll
      for (int i = 0; i < 8; ++i) reinterpret_cast<f32x4*>(vs + pl * D + sub * 32)[i] = vr[i];
    }
    float sj[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const f32x4* qv = reinterpret_cast<const f32x4*>(qs + j * D + sub * 32);
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f32x4 b = qv[i];
        a = fmaf(kr[i].x, b.x, a);
        a = fmaf(kr[i].y, b.y, a);
        a = fmaf(kr[i].z, b.z, a);
        a = fmaf(kr[i].w, b.w, a);
      }
      sj[j] = group_sum<4>(a);
    }
    if (sub == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) ps[j * TP + pl] = pl < n ? sj[j] * scale : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < HPW; ++r) {
      const int j = wave + 4 * r;
      if (j < G) {
        const float s = ps[j * TP + lane];
        const float mn = fmaxf(M[r], wave_max(s));
        const float p = __expf(s - mn);
        const float c = __expf(M[r] - mn);
        L[r] = L[r] * c + wave_sum(p);
        M[r] = mn;
        ps[j * TP + lane] = p;
        if (lane == 0) cs[j] = c;
      }
    }
    __syncthreads();
    if (QUAD) {
      f32x4 a = acc4 * cs[hq];
      const float* pj = ps + hq * TP;
      for (int p = 0; p < n; ++p) a += pj[p] * *reinterpret_cast<const f32x4*>(vs + p * D + 4 * dq);
      acc4 = a;
    } else {
#pragma unroll
      for (int i = 0; i < JPT; ++i) {
        const int j = G >= 2 ? jh + 2 * i : 0;
        if (G >= 2 || jh == 0) {
          float a = acc[i] * cs[j];
          const float* pj = ps + j * TP;
          for (int p = 0; p < n; ++p) a = fmaf(pj[p], vs[p * D + dd], a);
          acc[i] = a;
        }
      }
    }
  }
  float* base = part + ((size_t)g * G * S + sp) * (D + 2);
  if (QUAD) {
    float* o = base + (size_t)hq * S * (D + 2) + 2 + 4 * dq;
    o[0] = acc4.x;
    o[1] = acc4.y;
    o[2] = acc4.z;
    o[3] = acc4.w;
  } else {
#pragma unroll
    for (int i = 0; i < JPT; ++i) {
      const int j = G >= 2 ? jh + 2 * i : 0;
      if (G >= 2 || jh == 0) base[(size_t)j * S * (D + 2) + 2 + dd] = acc[i];
    }
  }
#pragma unroll
  for (int r = 0; r < HPW; ++r) {
    const int j = wave + 4 * r;
    if (j < G && lane == 0) {
      base[(size_t)j * S * (D + 2)] = M[r];
      base[(size_t)j * S * (D + 2) + 1] = L[r];
    }
  }
}

// ---------------------------------------------------------------------------
// The same split-K decode attention for G = 8 query heads per kv head, with a
// tile layout that keeps the operands of both products in registers.  Lane
// bits 0, 1, 4, 5 give the dim group dg (dims 4 dg .. + 3 and 64 + 4 dg ..
// + 3), lane bits 2, 3 and the wave give the position group pg (positions
// pg, pg + 16, pg + 32, pg + 48 of a 64-position tile).  A thread holds its
// 8 dims of q for all 8 heads, and of K and V for its 4 positions:
//   * QK: 8 heads x 4 positions partial dots over 8 dims, then a reduce-
//     scatter over the 16 dim groups (row swaps over lane bits 5 and 4, DPP
//     over bits 1 and 0) leaves each lane 2 complete scores;
//   * softmax per head as in the generic kernel (one position per lane);
//   * PV: o[8 heads][8 dims] += p * V from the thread's own V registers, the
//     probabilities read as [position][head] rows;
// and at the split's end the 16 position groups' partial outputs are added
// (DPP within a wave, then the 4 waves through LDS, in a fixed order).  The
// next tile's K is requested after QK and its V after PV, as buffer loads
// bounded by the split (zeros past it).

// Reduce-scatter step over lane bit 5 (d = 32) or 4 (d = 16) with the gfx950
// row swaps: lanes with the bit clear return a + a of the partner lane, lanes
// with it set b + b of the partner.
template <int d>
__device__ __forceinline__ float swap_add(float a, float b) {
  const auto r = d == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same step over lane bit 1 (CTRL = xor 2) or 0 (xor 1) through DPP.
template <int CTRL>
__device__ __forceinline__ float quad_add(float a, float b, bool bit) {
  return (bit ? b : a) + dpp_f<CTRL>(bit ? a : b);
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b, float c) {
  c = fmaf(a.x, b.x, c);
  c = fmaf(a.y, b.y, c);
  c = fmaf(a.z, b.z, c);
  return fmaf(a.w, b.w, c);
}

// A buffer record over `bytes` bytes at `base` (both the same in every lane;
// taken from lane 0 so the record lives in scalar registers rather than being
// rebuilt lane by lane around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t kv_record(const void* base, int bytes) {
  const uint64_t v = (uint64_t)base;
  const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 4 values of one K or V row at byte offset `off` of the split's record
template <typename KVT>
__device__ __forceinline__ f32x4 kv_load4(__amdgpu_buffer_rsrc_t r, int off) {
  if constexpr (sizeof(KVT) == 4) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else {
    const u32x2 a = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    return f32x4{bf16_lo(a.x), bf16_hi(a.x), bf16_lo(a.y), bf16_hi(a.y)};
  }
}

// dot of 8 bf16 (one 16-byte piece of a B row) with 8 floats
__device__ __forceinline__ float dot8_bf16(u32x4 w, f32x4 u0, f32x4 u1) {
  float a = 0.f;
  a = fmaf(bf16_lo(w.x), u0.x, a);
  a = fmaf(bf16_hi(w.x), u0.y, a);
  a = fmaf(bf16_lo(w.y), u0.z, a);
  a = fmaf(bf16_hi(w.y), u0.w, a);
  a = fmaf(bf16_lo(w.z), u1.x, a);
  a = fmaf(bf16_hi(w.z), u1.y, a);
  a = fmaf(bf16_lo(w.w), u1.z, a);
  a = fmaf(bf16_hi(w.w), u1.w, a);
  return a;
}

// One row of an adapter's up product, B[row] . u over r columns.  Rows of B
// are r bf16 apart, so they are 16-byte aligned only when r is a multiple of
// 8: then the first NPRE 8-column pieces come from registers loaded ahead and
// the rest are read here in pieces; any other r is read value by value.
template <int NPRE>
__device__ __forceinline__ float lora_row(const u32x4* pre, const f32x4* upre, const uint16_t* brow, const float* u,
                                          int r) {
  float a = 0.f;
  if ((r & 7) == 0) {
#pragma unroll
    for (int c = 0; c < NPRE; ++c)
      if (8 * c < r) a += dot8_bf16(pre[c], upre[2 * c], upre[2 * c + 1]);
    for (int k0 = 8 * NPRE; k0 < r; k0 += 8)
      a += dot8_bf16(*reinterpret_cast<const u32x4*>(brow + k0), *reinterpret_cast<const f32x4*>(u + k0),
                     *reinterpret_cast<const f32x4*>(u + k0 + 4));
  } else {
    for (int k = 0; k < r; ++k) a = fmaf(bf16_to_f(brow[k]), u[k], a);
  }
  return a;
}

// One head of the new row from registers (lane: dims lane and lane + 64):
// optional RMSNorm over the head's D values (gain), then RoPE with the
// half-split pairing (j, j + D/2); the results go to out[lane], out[lane + 64].
__device__ __forceinline__ void norm_rope_regs(float a, float b, bool gain, float ga, float gb, float eps, float c,
                                               float s, float* out) {
  const int l = threadIdx.x & 63;
  if (gain) {
    const float r = 1.0f / sqrtf(wave_sum(a * a + b * b) / (float)D + eps);
    a = a * r * ga;
    b = b * r * gb;
  }
  out[l] = a * c - b * s;
  out[l + 64] = b * c + a * s;
}

// Row stride (floats) of the waves' partial outputs in LDS: 64 values and 4 of
// padding, so that the 16 rows written or read at once fall on distinct banks.
constexpr int kOredStride = 68;

template <bool LORA, typename KVT>
__global__ __launch_bounds__(256) void k_attn_decode8(const float* __restrict__ qkv, const float* __restrict__ qn,
                                                      const float* __restrict__ kn, float eps,
                                                      const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                                                      KVT* __restrict__ Kc, KVT* __restrict__ Vc, int max_pos,
                                                      const DevState* __restrict__ st, int row, int S, int cmin, float scale,
                                                      float* __restrict__ part, LoraUp lu) {
  constexpr int G = 8;
  const int g = blockIdx.x, sp = blockIdx.y;

  __shared__ __align__(16) float qs[G * D];
  __shared__ __align__(16) float ps[G * TP];  // scores [head][position]
  __shared__ __align__(16) float pt[TP * G];  // probabilities [position][head]
  __shared__ __align__(16) float cs[G];       // per-head rescale of this tile
  __shared__ __align__(16) float kv_new[2 * D];
  __shared__ __align__(16) float ored[4 * 16 * kOredStride];  // the waves' partial outputs

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const float* grp = qkv + (size_t)g * (G + 2) * D;

  // ---- 1. what the q side reads that does not depend on the step's position
  // (lane: dims lane and lane + 64 of q heads wave and wave + 4; wave 3 also
  // of the new k and v), requested first: the step state is read after it and
  // the K/V rows after both, so that no wait for one waits for a later one
  float qa[2], qb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + 4 * i;
    qa[i] = grp[j * D + lane];
    qb[i] = grp[j * D + lane + 64];
  }
  float ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
  if (wave == 3) {
    ka = grp[G * D + lane];
    kb = grp[G * D + lane + 64];
    va = grp[(G + 1) * D + lane];
    vb = grp[(G + 1) * D + lane + 64];
  }
  const float gq0 = qn ? qn[lane] : 1.f, gq1 = qn ? qn[lane + 64] : 1.f;
  const float gk0 = kn ? kn[lane] : 1.f, gk1 = kn ? kn[lane + 64] : 1.f;
  // adapter (q += s B_q u_q, v += s B_v u_v, "EMBERGLASS (qwen-webgpu-lora)
  // README", LoRA sections): with r a multiple of 8, the first 16 columns of
  // this lane's B rows and of u, ahead
  constexpr int NPRE = LORA ? 2 : 1;
  u32x4 bqa[2][NPRE], bqb[2][NPRE], bva[NPRE], bvb[NPRE];
  f32x4 uq[2 * NPRE], uv[2 * NPRE];
  const int r = lu.r;
  const bool r8 = (r & 7) == 0;
  int zoff = 0;
  asm volatile("" : "+v"(zoff));  // (u through a per-lane address: vector loads, no scalar wait)
  const float* uu = lu.u + zoff;
  if (LORA && r8) {
#pragma unroll
    for (int c = 0; c < NPRE; ++c) {
      if (8 * c < r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const size_t row = (size_t)(g * G + wave + 4 * i) * D + lane;
          bqa[i][c] = *reinterpret_cast<const u32x4*>(lu.bq + row * r + 8 * c);
          bqb[i][c] = *reinterpret_cast<const u32x4*>(lu.bq + (row + 64) * r + 8 * c);
        }
        if (wave == 3) {
          bva[c] = *reinterpret_cast<const u32x4*>(lu.bv + ((size_t)g * D + lane) * r + 8 * c);
          bvb[c] = *reinterpret_cast<const u32x4*>(lu.bv + ((size_t)g * D + lane + 64) * r + 8 * c);
        }
        uq[2 * c] = *reinterpret_cast<const f32x4*>(uu + 8 * c);
        uq[2 * c + 1] = *reinterpret_cast<const f32x4*>(uu + 8 * c + 4);
        uv[2 * c] = *reinterpret_cast<const f32x4*>(uu + r + 8 * c);
        uv[2 * c + 1] = *reinterpret_cast<const f32x4*>(uu + r + 8 * c + 4);
      }
    }
  }

  // ---- the split and what depends on the position.  A split past the
  // context holds no position: an empty record, no tile, and a partial the
  // merge does not read.
  const int ctx = st->pos + row + 1, pos = ctx - 1;  // (row: of a batch of new rows)
  const int C = split_len(ctx, S, cmin);
  const int p_begin = sp * C;
  const int p_end = max(p_begin, min(p_begin + C, ctx));
  const bool owns_new = p_begin < ctx && p_end == ctx;
  const bool kvw = owns_new && wave == 3;  // wave 3 finishes the new row's k and v
  const float cth = cos_t[(size_t)pos * (D / 2) + lane], sth = sin_t[(size_t)pos * (D / 2) + lane];

  // ---- 2. the split's first tile of K and V rows
  const int dg = (lane & 3) | ((lane >> 4) << 2);
  const int pg = wave * 4 + ((lane >> 2) & 3);
  const int kv_bytes = (p_end - p_begin) * D * (int)sizeof(KVT);
  const __amdgpu_buffer_rsrc_t rk = kv_record(Kc + ((size_t)g * max_pos + p_begin) * D, kv_bytes);
  const __amdgpu_buffer_rsrc_t rv = kv_record(Vc + ((size_t)g * max_pos + p_begin) * D, kv_bytes);
  const int esz = (int)sizeof(KVT);
  // byte offset of (tile-relative row rr, half h) in the split's record
  auto off = [&](int rr, int h) { return (rr * D + 64 * h + 4 * dg) * esz; };
  f32x4 kk[4][2], vv[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) kk[i][h] = kv_load4<KVT>(rk, off(pg + 16 * i, h));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) vv[i][h] = kv_load4<KVT>(rv, off(pg + 16 * i, h));

  // ---- 3. q heads (adapter, QK-norm, RoPE) into LDS; the new k and v
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = wave + 4 * i;
    float a = qa[i], b = qb[i];
    if (LORA) {
      const uint16_t* b0 = lu.bq + ((size_t)(g * G + j) * D + lane) * r;
      a += lu.scale * lora_row<NPRE>(bqa[i], uq, b0, lu.u, r);
      b += lu.scale * lora_row<NPRE>(bqb[i], uq, b0 + 64 * (size_t)r, lu.u, r);
    }
    norm_rope_regs(a, b, qn != nullptr, gq0, gq1, eps, cth, sth, qs + j * D);
  }
  if (kvw) {
    if (LORA) {
      const uint16_t* b0 = lu.bv + ((size_t)g * D + lane) * r;
      va += lu.scale * lora_row<NPRE>(bva, uv, b0, lu.u + r, r);
      vb += lu.scale * lora_row<NPRE>(bvb, uv, b0 + 64 * (size_t)r, lu.u + r, r);
    }
    norm_rope_regs(ka, kb, kn != nullptr, gk0, gk1, eps, cth, sth, kv_new);
    // the new row as the cache stores it (bf16 cache: rounded), for this step too
    const float k0 = kv_round<KVT>(kv_new[lane]), k1 = kv_round<KVT>(kv_new[lane + 64]);
    const float v0 = kv_round<KVT>(va), v1 = kv_round<KVT>(vb);
    kv_new[lane] = k0;
    kv_new[lane + 64] = k1;
    kv_new[D + lane] = v0;
    kv_new[D + 64 + lane] = v1;
    KVT* kr = Kc + ((size_t)g * max_pos + pos) * D;
    KVT* vr = Vc + ((size_t)g * max_pos + pos) * D;
    st_kv(kr + lane, k0);
    st_kv(kr + lane + 64, k1);
    st_kv(vr + lane, v0);
    st_kv(vr + lane + 64, v1);
  }

  const bool b0 = lane & 1, b1 = lane & 2;
  const int isel = (lane >> 4) & 3;  // which of the lane's 4 positions its two final scores belong to
  const int jsel = 4 * (int)b1 + 2 * (int)b0;  // and their heads: jsel, jsel + 1
  __syncthreads();  // q and the new row staged
  f32x4 qq[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) qq[j][h] = *reinterpret_cast<const f32x4*>(qs + j * D + 64 * h + 4 * dg);
  f32x4 acc[G][2];
#pragma unroll
  for (int j = 0; j < G; ++j) acc[j][0] = acc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float M[2], L[2];
  M[0] = M[1] = -INFINITY;
  L[0] = L[1] = 0.f;

  for (int t0 = p_begin; t0 < p_end; t0 += TP) {
    const int n = min(TP, p_end - t0);
    if (owns_new) {  // the new row: from LDS, not the cache
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (t0 + pg + 16 * i == pos) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            kk[i][h] = *reinterpret_cast<const f32x4*>(kv_new + 64 * h + 4 * dg);
            vv[i][h] = *reinterpret_cast<const f32x4*>(kv_new + D + 64 * h + 4 * dg);
          }
        }
      }
    }
    // ---- scores: partial dots, then the reduce-scatter over the dim groups
    float sc[32];  // [position i][head j] = sc[8 i + j]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < G; ++j) sc[8 * i + j] = dot4(kk[i][1], qq[j][1], dot4(kk[i][0], qq[j][0], 0.f));
    const int tn = t0 + TP - p_begin;  // the next tile's first row in the record
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) kk[i][h] = kv_load4<KVT>(rk, off(tn + pg + 16 * i, h));
    float r1[16], r2[8], r3[4];
#pragma unroll
    for (int k = 0; k < 16; ++k) r1[k] = swap_add<32>(sc[k], sc[k + 16]);
#pragma unroll
    for (int k = 0; k < 8; ++k) r2[k] = swap_add<16>(r1[k], r1[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) r3[k] = quad_add<kDppQuadSwap2>(r2[k], r2[k + 4], b1);
    const float s0 = quad_add<kDppQuadSwap1>(r3[0], r3[2], b0);
    const float s1 = quad_add<kDppQuadSwap1>(r3[1], r3[3], b0);
    {
      const int pr = pg + 16 * isel;
      const bool ok = pr < n;
      ps[jsel * TP + pr] = ok ? s0 * scale : -INFINITY;
      ps[(jsel + 1) * TP + pr] = ok ? s1 * scale : -INFINITY;
    }
    __syncthreads();
    // ---- online softmax, heads wave and wave + 4 (one position per lane)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int j = wave + 4 * rr;
      const float sv = ps[j * TP + lane];
      const float mn = fmaxf(M[rr], wave_max(sv));
      const float p = __expf(sv - mn);
      const float c = __expf(M[rr] - mn);
      L[rr] = L[rr] * c + wave_sum(p);
      M[rr] = mn;
      pt[lane * G + j] = p;
      if (lane == 0) cs[j] = c;
    }
    __syncthreads();
    // ---- PV from the thread's own V rows
    {
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cs), c1 = *reinterpret_cast<const f32x4*>(cs + 4);
      const float cj[G] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int j = 0; j < G; ++j) {
        acc[j][0] *= cj[j];
        acc[j][1] *= cj[j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* pp = pt + (pg + 16 * i) * G;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(pp), p1 = *reinterpret_cast<const f32x4*>(pp + 4);
        const float pj[G] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int j = 0; j < G; ++j) {
          acc[j][0] += pj[j] * vv[i][0];
          acc[j][1] += pj[j] * vv[i][1];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) vv[i][h] = kv_load4<KVT>(rv, off(tn + pg + 16 * i, h));
  }

  // ---- the 16 position groups' outputs: the 4 of a wave by DPP (row
  // rotations by 8 and 4 stay on lanes with the same dim group), then the
  // waves in order through LDS
  __syncthreads();  // the adapter scratch is no longer read
#pragma unroll
  for (int j = 0; j < G; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 v = acc[j][h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = v[e];
        x += dpp_f<0x128>(x);  // row_ror:8
        x += dpp_f<0x124>(x);  // row_ror:4
        v[e] = x;
      }
      acc[j][h] = v;
    }
  }
  if (((lane >> 2) & 3) == 0) {
    float* dst = ored + (wave * 16 + dg) * kOredStride;
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) *reinterpret_cast<f32x4*>(dst + j * 8 + h * 4) = acc[j][h];
  }
  __syncthreads();
  float* base = part + ((size_t)g * G * S + sp) * (D + 2);
  {
    const int j = tid >> 5, d0 = (tid & 31) * 4;  // head j, dims d0 .. d0 + 3
    const int h = d0 >> 6, dgo = (d0 & 63) >> 2;
    f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) o += *reinterpret_cast<const f32x4*>(ored + (w * 16 + dgo) * kOredStride + j * 8 + h * 4);
    float* dst = base + (size_t)j * S * (D + 2) + 2 + d0;
    dst[0] = o.x;
    dst[1] = o.y;
    dst[2] = o.z;
    dst[3] = o.w;
  }
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int j = wave + 4 * rr;
    if (lane == 0) {
      base[(size_t)j * S * (D + 2)] = M[rr];
      base[(size_t)j * S * (D + 2) + 1] = L[rr];
    }
  }
}

// o_h = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M} over the splits that hold
// positions.  grid (nq, D / 32), block 256: 32 dims x 8 split classes (s mod 8).
// Every thread requests its splits' m, l and o in one go (indices clamped to
// the S written splits, so no load waits on the step state), keeps those
// that hold positions, and merges them in registers, 8 U splits per pass;
// the classes are then merged in class order.
constexpr int kMaxSplits = 1024;

// (m, l, o) <- the merge of (m, l, o) and (mc, lc, oc); a side with no
// position (m = -inf, l = o = 0) weighs e^-inf = 0, with no branch.
__device__ __forceinline__ void merge_into(float& m, float& l, float& o, float mc, float lc, float oc) {
  const float mn = fmaxf(m, mc), mr = fmaxf(mn, -3.0e38f);
  const float a = __expf(m - mr), b = __expf(mc - mr);
  l = l * a + lc * b;
  o = o * a + oc * b;
  m = mn;
}

__global__ __launch_bounds__(256) void k_attn_merge_decode(const float* __restrict__ part, int S, int cmin,
                                                           const DevState* __restrict__ st, int row,
                                                           float* __restrict__ o_out) {
  constexpr int U = 16;
  __shared__ float mm[8], ll[8], oo[8][33];
  const int h = blockIdx.x, tid = threadIdx.x, nqh = gridDim.x;
  const int d = blockIdx.y * 32 + (tid & 31), sg = tid >> 5;
  // (grid z: the rows of a batch, their partials and outputs one after the
  // other; the split geometry is that of the batch's last row, `row`)
  part += (size_t)blockIdx.z * nqh * S * (D + 2);
  o_out += (size_t)blockIdx.z * nqh * D;
  const float* base = part + (size_t)h * S * (D + 2);
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8 * U) {  // uniform
    float mv[U], lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float* ps = base + (size_t)min(s0 + sg + 8 * u, S - 1) * (D + 2);
      mv[u] = ps[0];
      lv[u] = ps[1];
      ov[u] = ps[2 + d];
    }
    // (read here, after the loads are requested: the step state is not
    // waited for before them)
    const int ctx = *reinterpret_cast<const volatile int*>(&st->pos) + row + 1;
    const int C = split_len(ctx, S, cmin);
    const int s_act = min(S, (ctx + C - 1) / C);
    float mc = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + sg + 8 * u >= s_act) {  // a split with no position: its words are stale, not read
        mv[u] = -INFINITY;
        lv[u] = ov[u] = 0.f;
      }
      mc = fmaxf(mc, mv[u]);
    }
    float lc = 0.f, oc = 0.f;
    const float mref = fmaxf(mc, -3.0e38f);  // finite: a masked split weighs e^-inf = 0, with no branch
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = __expf(mv[u] - mref);
      lc = fmaf(lv[u], e, lc);
      oc = fmaf(ov[u], e, oc);
    }
    merge_into(m, l, o, mc, lc, oc);
  }
  if ((tid & 31) == 0) {
    mm[sg] = m;
    ll[sg] = l;
  }
  oo[sg][tid & 31] = o;
  __syncthreads();
  if (sg == 0) {
    float M = mm[0], L = ll[0], O = oo[0][tid];
#pragma unroll
    for (int k = 1; k < 8; ++k) merge_into(M, L, O, mm[k], ll[k], oo[k][tid]);
    o_out[(size_t)h * D + d] = O / L;
  }
}

// The bf16 halves of v (as the projection input split makes them).
__device__ __forceinline__ void store_hilo_o(uint16_t* __restrict__ h, uint16_t* __restrict__ l, size_t i, float v) {
  const uint32_t hb = bf16_rne(v);
  h[i] = (uint16_t)hb;
  l[i] = (uint16_t)bf16_rne(v - __uint_as_float(hb << 16));
}

// The batch attention's split partials merged: one thread per (row, head,
// dim), over all S splits (every split's partials are written, those with no
// visible position as m = -inf, l = o = 0), in split order.
__global__ __launch_bounds__(256) void k_attn_merge_rows(const float* __restrict__ part, int S, int total,
                                                         float* __restrict__ o_out, uint16_t* __restrict__ oh,
                                                         uint16_t* __restrict__ ol) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int d = i % D, th = i / D;  // th = row nq + head
  const float* base = part + (size_t)th * S * (D + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < S; ++sp) M = fmaxf(M, base[(size_t)sp * (D + 2)]);
  float L = 0.f, O = 0.f;
  for (int sp = 0; sp < S; ++sp) {
    const float* ps = base + (size_t)sp * (D + 2);
    const float e = __expf(ps[0] - M);
    L = fmaf(ps[1], e, L);
    O = fmaf(ps[2 + d], e, O);
  }
  const float o = O / L;
  o_out[(size_t)th * D + d] = o;
  if (oh) store_hilo_o(oh, ol, (size_t)th * D + d, o);  // (optional: the o_proj input halves too)
}

// ---------------------------------------------------------------------------
// Causal attention for a prefill of T >= 2 rows (flash style).  Query row t
// sits at position pos + t (pos = the step state's position) and sees cache
// positions 0 .. pos + t, its own included.  S = Q K^T and O += P V are dense
// contractions per tile, so they run as v_mfma_f32_16x16x32_bf16 with
// every f32 operand split into bf16 halves (x = hi + lo, both rounded to
// nearest even) and three products (hi.hi + hi.lo + lo.hi, the lo.lo term is
// below f32 rounding of the result); accumulation is f32.
//
// grid (nkv, ceil(T / (16 NW / G))), block 64 NW (NW = 4 waves, or 8 for
// long batches: the same K/V tile then serves twice the queries).  Split form (SPLIT,
// short batches at long contexts): grid (nkv, ceil(T / (64 / G)) S), the
// positions 0 .. pos + T - 1 cut into S splits of split_len(pos + T, S, cmin)
// as the decode attention cuts them, and each block writes the partials
// {m, l, o} of its query vectors over its split (part[(row nq + head) S +
// split]) for k_attn_merge_decode.  A block owns 16 NW query
// vectors of kv head g; wave w owns 16 of them (the A operand of S, kept in
// registers for the whole kernel).  Per tile of 32 cache positions the block
// stages K (row-major) and V (transposed) as bf16 halves in LDS; each wave
// forms its 16 x 32 score tile, updates the online softmax of its rows
// (row maxima and sums over the 16 lanes that hold a row, by DPP; base-2
// exponentials with log2 e folded into the query scale; the causal and range
// masks only on tiles that reach them; the output rescale skipped when no
// row maximum of the wave moved), writes
// P's halves to its own LDS slice in the A-operand layout, and accumulates
// its 16 x 128 output tile.
template <int G, typename KVT, bool SPLIT, int NW = 4>
__global__ __launch_bounds__(64 * NW) void k_attn_prefill_mfma(const float* __restrict__ q, int T, int nq,
                                                           const KVT* __restrict__ Kc,
                                                           const KVT* __restrict__ Vc, int max_pos,
                                                           const DevState* __restrict__ st, float scale,
                                                           float* __restrict__ o_out, int ldo, int S, int cmin,
                                                           float* __restrict__ part, uint16_t* __restrict__ oh,
                                                           uint16_t* __restrict__ ol) {
  constexpr int QV = 16 * NW, R = QV / G, BK = 32;
  constexpr int PPT = 4 * 4 / NW, PG = BK / PPT;  // staging: positions per thread, position groups
  constexpr int KS = D + 8;   // K row stride (bf16)
  constexpr int VS = BK + 8;  // V^T row stride (bf16)
  constexpr int PS = BK + 8;  // P row stride (bf16)
  __shared__ __align__(16) uint16_t Kh[BK * KS], Kl[BK * KS];
  __shared__ __align__(16) uint16_t Vth[D * VS], Vtl[D * VS];
  __shared__ __align__(16) uint16_t Ph[NW][16 * PS], Pl[NW][16 * PS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;  // fragment row / column, k-quarter
  const int g = blockIdx.x;
  const int tile = SPLIT ? blockIdx.y / S : gridDim.y - 1 - blockIdx.y, sp = SPLIT ? blockIdx.y % S : 0;
  const int t0 = tile * R;
  const int pos0 = st->pos;
  const int nrows = min(R, T - t0);
  const int kv_end = pos0 + t0 + nrows;  // one past the last row's position
  // positions of this block: all it sees, or its split of the batch's positions
  int k_begin = 0, k_end = kv_end;
  if (SPLIT) {
    const int C = split_len(pos0 + T, S, cmin);
    k_begin = min(sp * C, kv_end);
    k_end = min(sp * C + C, kv_end);
  }

  // this lane's query fragment: vector wave*16 + lr, dims 32 ks + 8 lq .. + 8,
  // scaled by scale log2 e so that the scores are in base-2 exponent units
  const float qscale = scale * 1.44269504088896341f;
  bf16x8 qh[4], ql[4];
  {
    const int v = wave * 16 + lr, r = v / G, j = v % G;
    const float* src = q + ((size_t)(t0 + r) * nq + g * G + j) * D + 8 * lq;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, b = a;
      if (r < nrows) {
        a = *reinterpret_cast<const f32x4*>(src + 32 * ks) * qscale;
        b = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4) * qscale;
      }
      uint32_t h[4], lo[4];
      split_bf16x2(a.x, a.y, h[0], lo[0]);
      split_bf16x2(a.z, a.w, h[1], lo[1]);
      split_bf16x2(b.x, b.y, h[2], lo[2]);
      split_bf16x2(b.z, b.w, h[3], lo[3]);
      qh[ks] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
      ql[ks] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], lo[2], lo[3]});
    }
  }
  // softmax state of this lane's 4 rows (rows 4 lq + e of the wave's 16)
  float m[4], l[4];
  int qpos[4];
  bool live[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = (wave * 16 + 4 * lq + e) / G;
    m[e] = -INFINITY;
    l[e] = 0.f;
    live[e] = r < nrows;
    qpos[e] = pos0 + t0 + r;
  }
  f32x4 oacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const KVT* Kg = Kc + (size_t)g * max_pos * D;
  const KVT* Vg = Vc + (size_t)g * max_pos * D;
  // staging map: positions PPT p4 .. + PPT - 1, dims 4 c4 .. + 3
  const int p4 = tid % PG, c4 = tid / PG;

  // a tile's K and V rows are requested while the previous tile is computed
  f32x4 kr[PPT], vr[PPT];
  auto load_tile = [&](int k0) {
    const int nk = min(BK, k_end - k0);
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int p = PPT * p4 + pp;
      kr[pp] = vr[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p < nk) {
        kr[pp] = ld_kv4(Kg + (size_t)(k0 + p) * D + 4 * c4);
        vr[pp] = ld_kv4(Vg + (size_t)(k0 + p) * D + 4 * c4);
      }
    }
  };
  if (k_begin < k_end) load_tile(k_begin);
  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
    const int nk = min(BK, k_end - k0);
    __syncthreads();  // the previous tile's K, V and P are consumed
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      uint32_t h[2], lo[2];
      split_bf16x2(kr[pp].x, kr[pp].y, h[0], lo[0]);
      split_bf16x2(kr[pp].z, kr[pp].w, h[1], lo[1]);
      *reinterpret_cast<u32x2*>(&Kh[(PPT * p4 + pp) * KS + 4 * c4]) = u32x2{h[0], h[1]};
      *reinterpret_cast<u32x2*>(&Kl[(PPT * p4 + pp) * KS + 4 * c4]) = u32x2{lo[0], lo[1]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // dim 4 c4 + i: its PPT positions, transposed
      uint32_t h[PPT / 2], lo[PPT / 2];
#pragma unroll
      for (int pp = 0; pp < PPT; pp += 2) split_bf16x2(vr[pp][i], vr[pp + 1][i], h[pp / 2], lo[pp / 2]);
      if constexpr (PPT == 4) {
        *reinterpret_cast<u32x2*>(&Vth[(4 * c4 + i) * VS + 4 * p4]) = u32x2{h[0], h[1]};
        *reinterpret_cast<u32x2*>(&Vtl[(4 * c4 + i) * VS + 4 * p4]) = u32x2{lo[0], lo[1]};
      } else {
        *reinterpret_cast<uint32_t*>(&Vth[(4 * c4 + i) * VS + PPT * p4]) = h[0];
        *reinterpret_cast<uint32_t*>(&Vtl[(4 * c4 + i) * VS + PPT * p4]) = lo[0];
      }
    }
    if (k0 + BK < k_end) load_tile(k0 + BK);  // (kr, vr are staged: free)
    __syncthreads();
    // S = Q K^T: 16 queries x 32 positions (two 16 x 16 tiles)
    f32x4 sc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      sc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = (nt * 16 + lr) * KS + 32 * ks + 8 * lq;
        const bf16x8 kh = *reinterpret_cast<const bf16x8*>(&Kh[off]);
        const bf16x8 kl = *reinterpret_cast<const bf16x8*>(&Kl[off]);
        sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], kh, sc[nt], 0, 0, 0);
        sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], kl, sc[nt], 0, 0, 0);
        sc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks], kh, sc[nt], 0, 0, 0);
      }
    }
    // online softmax in base 2 (the scores carry log2 e); element e of
    // sc[nt] is row 4 lq + e, position nt * 16 + lr.  Masks only on a tile
    // that reaches past the block's first query position or the range end.
    const bool edge = nk < BK || k0 + BK - 1 > pos0 + t0;
    float cs[4];
    bool moved = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float s0 = sc[0][e], s1 = sc[1][e];
      if (edge) {
        if (!live[e] || lr >= nk || k0 + lr > qpos[e]) s0 = -INFINITY;
        if (!live[e] || 16 + lr >= nk || k0 + 16 + lr > qpos[e]) s1 = -INFINITY;
      }
      const float mn = fmaxf(m[e], group_max<16>(fmaxf(s0, s1)));
      const float mref = mn == -INFINITY ? 0.f : mn;  // a row with nothing visible yet
      const float e0 = __builtin_amdgcn_exp2f(s0 - mref), e1 = __builtin_amdgcn_exp2f(s1 - mref);
      const float c = __builtin_amdgcn_exp2f(m[e] - mref);
      l[e] = l[e] * c + group_sum<16>(e0 + e1);
      moved |= mn != m[e];
      m[e] = mn;
      cs[e] = c;
      uint32_t h, lo;  // (e0 in the low halves, e1 in the high)
      split_bf16x2(e0, e1, h, lo);
      uint16_t* ph = &Ph[wave][(4 * lq + e) * PS];
      uint16_t* pl = &Pl[wave][(4 * lq + e) * PS];
      ph[lr] = (uint16_t)h;
      ph[16 + lr] = (uint16_t)(h >> 16);
      pl[lr] = (uint16_t)lo;
      pl[16 + lr] = (uint16_t)(lo >> 16);
    }
    if (__any(moved)) {  // some row maximum of the wave moved: rescale (c = 1 elsewhere)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) oacc[dt][e] *= cs[e];
    }
    __syncthreads();  // P written (each wave reads back only its own slice)
    // O += P V: A = P (16 queries x 32 positions), B = V^T fragments of 8 dim tiles
    const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&Ph[wave][lr * PS + 8 * lq]);
    const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Pl[wave][lr * PS + 8 * lq]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int off = (dt * 16 + lr) * VS + 8 * lq;
      const bf16x8 vh = *reinterpret_cast<const bf16x8*>(&Vth[off]);
      const bf16x8 vl = *reinterpret_cast<const bf16x8*>(&Vtl[off]);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vh, oacc[dt], 0, 0, 0);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, vl, oacc[dt], 0, 0, 0);
      oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, vh, oacc[dt], 0, 0, 0);
    }
  }
  // element e of oacc[dt]: row 4 lq + e, dim dt * 16 + lr
  if (SPLIT) {  // the partials: m, l and o not divided by l
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = wave * 16 + 4 * lq + e, r = v / G, j = v % G;
      if (r < nrows) {
        float* dst = part + ((size_t)(t0 + r) * nq + g * G + j) * S * (D + 2) + (size_t)sp * (D + 2);
        if (lr == 0) {
          dst[0] = m[e] * 0.693147180559945309f;  // back to natural-log units for the merge
          dst[1] = l[e];
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) dst[2 + dt * 16 + lr] = oacc[dt][e];
      }
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int v = wave * 16 + 4 * lq + e, r = v / G, j = v % G;
    if (r < nrows) {
      const float inv = 1.0f / l[e];
      const size_t o0 = (size_t)(t0 + r) * ldo + (g * G + j) * D + lr;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const float o = oacc[dt][e] * inv;
        o_out[o0 + dt * 16] = o;
        if (oh) store_hilo_o(oh, ol, o0 + dt * 16, o);  // (optional: the o_proj input halves too)
      }
    }
  }
}

}  // namespace

int attn_decode_splits(int max_pos, int nkv, int ncu, int cmin) {
  int s = ncu / nkv;
  s = std::min(s, (max_pos + cmin - 1) / cmin);
  s = std::min(s, kMaxSplits);
  return std::max(s, 1);
}

void launch_attention_decode(hipStream_t s, const float* qkv, const float* qn, const float* kn, float eps,
                             const float* cos_t, const float* sin_t, int nq, int nkv, void* Kc, void* Vc,
                             int kv_bf16, int max_pos, const DevState* st, int S, int cmin, float* part, float* o_out,
                             const float* lora_u, const uint16_t* lora_bq, const uint16_t* lora_bv, int lora_r,
                             float lora_scale, int row) {
  const float scale = 1.0f / sqrtf((float)D);
  const dim3 grid(nkv, S);
  const LoraUp lu{lora_u, lora_bq, lora_bv, lora_r, lora_scale};
#define QD_ATTN_DECODE_T(G_, L_, T_)                                                                                 \
  if (G_ == 8)                                                                                                       \
    hipLaunchKernelGGL((k_attn_decode8<L_, T_>), grid, dim3(256), 0, s, qkv, qn, kn, eps, cos_t, sin_t, (T_*)Kc,    \
                       (T_*)Vc, max_pos, st, row, S, cmin, scale, part, lu);                                              \
  else                                                                                                               \
    hipLaunchKernelGGL((k_attn_decode<G_, L_, T_>), grid, dim3(256), 0, s, qkv, qn, kn, eps, cos_t, sin_t, (T_*)Kc, \
                       (T_*)Vc, max_pos, st, row, S, cmin, scale, part, lu)
#define QD_ATTN_DECODE(G_)                                     \
  if (kv_bf16) {                                               \
    if (lora_u) QD_ATTN_DECODE_T(G_, true, uint16_t);          \
    else QD_ATTN_DECODE_T(G_, false, uint16_t);                \
  } else {                                                     \
    if (lora_u) QD_ATTN_DECODE_T(G_, true, float);             \
    else QD_ATTN_DECODE_T(G_, false, float);                   \
  }
  switch (nq / nkv) {
    case 1: QD_ATTN_DECODE(1); break;
    case 2: QD_ATTN_DECODE(2); break;
    case 4: QD_ATTN_DECODE(4); break;
    case 8: QD_ATTN_DECODE(8); break;
    default: return;  // rejected by the host before any launch
  }
#undef QD_ATTN_DECODE
#undef QD_ATTN_DECODE_T
  hipLaunchKernelGGL(k_attn_merge_decode, dim3(nq, D / 32), dim3(256), 0, s, part, S, cmin, st, row, o_out);
}

void launch_attention_rows_split_only(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc,
                                      const void* Vc, int kv_bf16, int max_pos, const DevState* st, int S, int cmin,
                                      float* part);

int attn_prefill_splits(int T, int nq, int nkv, int ncu) {
  const int blocks = nkv * ((T + 64 / (nq / nkv) - 1) / (64 / (nq / nkv)));
  if (blocks >= ncu) return 1;
  return std::min(16, (2 * ncu + blocks - 1) / blocks);
}

void launch_attention_prefill(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc, const void* Vc,
                              int kv_bf16, int max_pos, const DevState* st, float* o_out, int ldo, int ncu,
                              float* part, int cmin, uint16_t* oh, uint16_t* ol) {
  const float scale = 1.0f / sqrtf((float)D);
  const int G = nq / nkv;
  const int S = part ? attn_prefill_splits(T, nq, nkv, ncu) : 1;
  if (S > 1 && ldo == nq * D) {  // fewer query tiles than CUs: the split form, then the merge
    launch_attention_rows_split_only(s, q, T, nq, nkv, Kc, Vc, kv_bf16, max_pos, st, S, cmin, part);
    const int total = T * nq * D;
    hipLaunchKernelGGL(k_attn_merge_rows, dim3((total + 255) / 256), dim3(256), 0, s, part, S, total, o_out, oh, ol);
    return;
  }
  // long batches: 8 waves (128 query vectors) per block while that still
  // leaves two blocks per CU, halving the K/V tiles staged per query
  const bool wide = nkv * ((T + 128 / G - 1) / (128 / G)) >= 2 * ncu;
  const int qv = wide ? 128 : 64;
  const dim3 grid(nkv, (T + qv / G - 1) / (qv / G)), block(wide ? 512 : 256);
#define QD_ATTN_PREFILL_NW(G_, NW_)                                                                                \
  if (kv_bf16)                                                                                                     \
    hipLaunchKernelGGL((k_attn_prefill_mfma<G_, uint16_t, false, NW_>), grid, block, 0, s, q, T, nq,              \
                       (const uint16_t*)Kc, (const uint16_t*)Vc, max_pos, st, scale, o_out, ldo, 1, 0, nullptr,     \
                       oh, ol);                                                                                     \
  else                                                                                                             \
    hipLaunchKernelGGL((k_attn_prefill_mfma<G_, float, false, NW_>), grid, block, 0, s, q, T, nq,                 \
                       (const float*)Kc, (const float*)Vc, max_pos, st, scale, o_out, ldo, 1, 0, nullptr, oh, ol)
#define QD_ATTN_PREFILL(G_)             \
  if (wide) {                           \
    QD_ATTN_PREFILL_NW(G_, 8);          \
  } else {                              \
    QD_ATTN_PREFILL_NW(G_, 4);          \
  }
  switch (G) {
    case 1: QD_ATTN_PREFILL(1); break;
    case 2: QD_ATTN_PREFILL(2); break;
    case 4: QD_ATTN_PREFILL(4); break;
    case 8: QD_ATTN_PREFILL(8); break;
    default: break;  // rejected by the host before any launch
  }
#undef QD_ATTN_PREFILL
#undef QD_ATTN_PREFILL_NW
}

void launch_attention_rows_split_only(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc,
                                      const void* Vc, int kv_bf16, int max_pos, const DevState* st, int S, int cmin,
                                      float* part) {
  const float scale = 1.0f / sqrtf((float)D);
  const int G = nq / nkv;
  const dim3 grid(nkv, ((T + 64 / G - 1) / (64 / G)) * S);
#define QD_ATTN_ROWS(G_)                                                                                           \
  if (kv_bf16)                                                                                                     \
    hipLaunchKernelGGL((k_attn_prefill_mfma<G_, uint16_t, true>), grid, dim3(256), 0, s, q, T, nq,                \
                       (const uint16_t*)Kc, (const uint16_t*)Vc, max_pos, st, scale, nullptr, 0, S, cmin, part,    \
                       nullptr, nullptr);                                                                           \
  else                                                                                                             \
    hipLaunchKernelGGL((k_attn_prefill_mfma<G_, float, true>), grid, dim3(256), 0, s, q, T, nq, (const float*)Kc,  \
                       (const float*)Vc, max_pos, st, scale, nullptr, 0, S, cmin, part, nullptr, nullptr)
  switch (G) {
    case 1: QD_ATTN_ROWS(1); break;
    case 2: QD_ATTN_ROWS(2); break;
    case 4: QD_ATTN_ROWS(4); break;
    case 8: QD_ATTN_ROWS(8); break;
    default: return;  // rejected by the host before any launch
  }
#undef QD_ATTN_ROWS
}

void launch_attention_rows_split(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc, const void* Vc,
                                 int kv_bf16, int max_pos, const DevState* st, int S, int cmin, float* part,
                                 float* o_out) {
  launch_attention_rows_split_only(s, q, T, nq, nkv, Kc, Vc, kv_bf16, max_pos, st, S, cmin, part);
  // the rows' merges (their split geometry: that of the last row)
  hipLaunchKernelGGL(k_attn_merge_decode, dim3(nq, D / 32, T), dim3(256), 0, s, part, S, cmin, st, T - 1, o_out);
}
