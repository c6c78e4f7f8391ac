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

template <int G>
__global__ __launch_bounds__(256) void k_attn_decode(const float* __restrict__ qkv, const float* __restrict__ qn,
                                                     const float* __restrict__ kn, float eps,
                                                     const float* __restrict__ cos_t, const float* __restrict__ sin_t,
                                                     float* __restrict__ Kc, float* __restrict__ Vc, int max_pos,
                                                     const DevState* __restrict__ st, int S, int cmin, float scale,
                                                     float* __restrict__ part) {
  const int g = blockIdx.x, sp = blockIdx.y;
  const int ctx = st->pos + 1, pos = ctx - 1;
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
  for (int j = wave; j < G; j += 4) norm_rope_head(grp + j * D, qn, eps, cos_t, sin_t, pos, qs + j * D);
  const bool owns_new = p_end == ctx;
  if (owns_new && wave == 3) {  // wave 3 has the fewest q heads
    norm_rope_head(grp + G * D, kn, eps, cos_t, sin_t, pos, kv_new);
    kv_new[D + lane] = grp[(G + 1) * D + lane];
    kv_new[D + 64 + lane] = grp[(G + 1) * D + 64 + lane];
    float* kr = Kc + ((size_t)g * max_pos + pos) * D;
    float* vr = Vc + ((size_t)g * max_pos + pos) * D;
    kr[lane] = kv_new[lane];
    kr[lane + 64] = kv_new[lane + 64];
    vr[lane] = kv_new[D + lane];
    vr[lane + 64] = kv_new[D + 64 + lane];
  }

  const int pl = tid >> 2, sub = tid & 3;  // load / score mapping: position, quarter of the dims
  const int dd = tid & 127, jh = tid >> 7; // output mapping: dim, head parity
  constexpr int JPT = G >= 2 ? G / 2 : 1;  // output heads per thread
  constexpr int HPW = G >= 4 ? G / 4 : 1;  // softmax heads per wave
  float acc[JPT];
#pragma unroll
  for (int i = 0; i < JPT; ++i) acc[i] = 0.f;
  float M[HPW], L[HPW];
#pragma unroll
  for (int r = 0; r < HPW; ++r) { M[r] = -INFINITY; L[r] = 0.f; }

  const float* Kg = Kc + (size_t)g * max_pos * D;
  const float* Vg = Vc + (size_t)g * max_pos * D;
  for (int t0 = p_begin; t0 < p_end; t0 += TP) {
    const int n = min(TP, p_end - t0);
    f32x4 kr[8], vr[8];
    const bool fresh = owns_new && t0 + pl == pos;  // the new row: from LDS, not the cache
    if (pl < n && !fresh) {
      const size_t off = (size_t)(t0 + pl) * D + sub * 32;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Kg + off) + i);
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Vg + off) + i);
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
  float* base = part + ((size_t)g * G * S + sp) * (D + 2);
#pragma unroll
  for (int i = 0; i < JPT; ++i) {
    const int j = G >= 2 ? jh + 2 * i : 0;
    if (G >= 2 || jh == 0) base[(size_t)j * S * (D + 2) + 2 + dd] = acc[i];
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

// o_h = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M} over the splits that hold
// positions, in split order.  grid (nq, D / 32), block 256: 32 dims x 8 split
// classes (s mod 8), summed in class order at the end.
constexpr int kMaxSplits = 1024;

__global__ __launch_bounds__(256) void k_attn_merge_decode(const float* __restrict__ part, int S, int cmin,
                                                           const DevState* __restrict__ st, float* __restrict__ o_out) {
  __shared__ float f[kMaxSplits];
  __shared__ float red[8];
  __shared__ float acc_s[8][33];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int ctx = st->pos + 1;
  const int C = split_len(ctx, S, cmin);
  const int s_act = min(S, (ctx + C - 1) / C);
  const float* base = part + (size_t)h * S * (D + 2);
  float m = -INFINITY;
  for (int s = tid; s < s_act; s += 256) m = fmaxf(m, base[(size_t)s * (D + 2)]);
  const float M = block_max_256(m, red);
  float lsum = 0.f;
  for (int s = tid; s < s_act; s += 256) {
    const float e = __expf(base[(size_t)s * (D + 2)] - M);
    f[s] = e;
    lsum = fmaf(base[(size_t)s * (D + 2) + 1], e, lsum);
  }
  const float Lt = block_sum_256(lsum, red);  // its barrier also publishes f[]
  const int d = blockIdx.y * 32 + (tid & 31), sg = tid >> 5;
  float a = 0.f;
#pragma unroll 4
  for (int s = sg; s < s_act; s += 8) a = fmaf(f[s], base[(size_t)s * (D + 2) + 2 + d], a);
  acc_s[sg][tid & 31] = a;
  __syncthreads();
  if (sg == 0) {
    float o = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) o += acc_s[k][tid & 31];
    o_out[(size_t)h * D + d] = o / Lt;
  }
}


// ---------------------------------------------------------------------------
// Causal attention for a prefill of T >= 2 rows (flash style, f32 on the VALU).
// Query row t sits at position pos + t (pos = the step state's position) and
// sees cache positions 0 .. pos + t, its own included.
//
// grid (nkv, ceil(T / (QV / G))), block 256.  A block owns kv head g and QV
// query vectors (QV / G consecutive rows times the G query heads of g), so a
// K/V tile in LDS serves all of them.  Per tile of BK = 2048 / QV positions:
//   scores: each thread forms a 2 (query) x 4 (position) tile of dot products
//           from LDS (queries pre-scaled by 1 / sqrt(d)); its positions are
//           kj + b BK / 4, so the lanes of a wave read consecutive K rows
//           (distinct LDS banks);
//   online softmax: the BK / 4 threads that share a query pair reduce the
//           tile's max and sum with DPP, rescale the running state and write
//           the probabilities (transposed) to LDS;
//   values: each thread accumulates a (QV / 8) (query) x 4 (dim) output tile.
// K and V of a tile share one LDS buffer (V is held in registers while the
// scores are formed), which keeps the block under 64 KiB of LDS.  QV = 32
// doubles the block count of short prompts.  Blocks with the longest causal
// ranges start first.
template <int G, int QV>
__global__ __launch_bounds__(256) void k_attn_prefill(const float* __restrict__ q, int T, int nq,
                                                      const float* __restrict__ Kc, const float* __restrict__ Vc,
                                                      int max_pos, const DevState* __restrict__ st, float scale,
                                                      float* __restrict__ o_out, int ldo) {
  constexpr int R = QV / G, BK = 2048 / QV, KG = BK / 4, QPT = QV / 8, RS = D + 4, PS = QV + 4;
  constexpr int VPT = BK * D / 4 / 256;  // V pieces per thread
  __shared__ __align__(16) float Qs[QV * RS];
  __shared__ __align__(16) float KVs[BK * RS];  // K of the tile, then its V
  __shared__ __align__(16) float Pt[BK * PS];  // probabilities [position][query]
  __shared__ float cs[QV];
  __shared__ float ls[QV];
  const int tid = threadIdx.x;
  const int g = blockIdx.x;
  const int t0 = (gridDim.y - 1 - blockIdx.y) * R;
  const int pos0 = st->pos;
  const int nrows = min(R, T - t0);
  const int kv_end = pos0 + t0 + nrows;  // one past the last row's position

  for (int i = tid; i < QV * D / 4; i += 256) {
    const int v = i / (D / 4), c4 = i % (D / 4), r = v / G, j = v % G;
    f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r < nrows) val = *reinterpret_cast<const f32x4*>(q + ((size_t)(t0 + r) * nq + g * G + j) * D + c4 * 4) * scale;
    *reinterpret_cast<f32x4*>(Qs + v * RS + c4 * 4) = val;
  }
  const int qi = tid / KG, kj = tid % KG;  // score mapping: queries 2 qi, 2 qi + 1; positions kj + KG b
  const int qg = tid >> 5, dg = tid & 31;  // value mapping: queries QPT qg .. + QPT - 1; dims 4 dg .. + 3
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  int qpos[2];
  bool live[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = (2 * qi + a) / G;
    live[a] = r < nrows;
    qpos[a] = pos0 + t0 + r;
  }
  f32x4 o[QPT];
#pragma unroll
  for (int a = 0; a < QPT; ++a) o[a] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* Kg = Kc + (size_t)g * max_pos * D;
  const float* Vg = Vc + (size_t)g * max_pos * D;

  for (int k0 = 0; k0 < kv_end; k0 += BK) {
    const int nk = min(BK, kv_end - k0);
    f32x4 vr[VPT];
    __syncthreads();  // queries staged; the previous tile consumed
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = tid + u * 256, p = i / (D / 4), c4 = i % (D / 4);
      f32x4 kv = f32x4{0.f, 0.f, 0.f, 0.f};
      vr[u] = kv;
      if (p < nk) {
        kv = *reinterpret_cast<const f32x4*>(Kg + (size_t)(k0 + p) * D + c4 * 4);
        vr[u] = *reinterpret_cast<const f32x4*>(Vg + (size_t)(k0 + p) * D + c4 * 4);
      }
      *reinterpret_cast<f32x4*>(KVs + p * RS + c4 * 4) = kv;
    }
    __syncthreads();
    float sc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) sc[a][b] = 0.f;
#pragma unroll 4
    for (int c = 0; c < D; c += 4) {
      const f32x4 qa = *reinterpret_cast<const f32x4*>(Qs + (2 * qi) * RS + c);
      const f32x4 qb = *reinterpret_cast<const f32x4*>(Qs + (2 * qi + 1) * RS + c);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(KVs + (kj + KG * b) * RS + c);
        sc[0][b] = fmaf(qa.x, kv.x, fmaf(qa.y, kv.y, fmaf(qa.z, kv.z, fmaf(qa.w, kv.w, sc[0][b]))));
        sc[1][b] = fmaf(qb.x, kv.x, fmaf(qb.y, kv.y, fmaf(qb.z, kv.z, fmaf(qb.w, kv.w, sc[1][b]))));
      }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      float tmax = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int pl = kj + KG * b;
        if (!live[a] || pl >= nk || k0 + pl > qpos[a]) sc[a][b] = -INFINITY;
        tmax = fmaxf(tmax, sc[a][b]);
      }
      tmax = group_max<KG>(tmax);
      const float mn = fmaxf(m[a], tmax);
      const float mref = mn == -INFINITY ? 0.f : mn;  // a query with nothing visible yet
      float ps = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float p = __expf(sc[a][b] - mref);
        Pt[(kj + KG * b) * PS + 2 * qi + a] = p;
        ps += p;
      }
      ps = group_sum<KG>(ps);
      const float c = __expf(m[a] - mref);
      l[a] = l[a] * c + ps;
      m[a] = mn;
      if (kj == 0) cs[2 * qi + a] = c;
    }
    __syncthreads();  // every score formed: the buffer takes V
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int i = tid + u * 256, p = i / (D / 4), c4 = i % (D / 4);
      *reinterpret_cast<f32x4*>(KVs + p * RS + c4 * 4) = vr[u];
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < QPT; ++a) o[a] = o[a] * cs[QPT * qg + a];
    for (int p = 0; p < nk; ++p) {
      const f32x4 vv = *reinterpret_cast<const f32x4*>(KVs + p * RS + 4 * dg);
#pragma unroll
      for (int a4 = 0; a4 < QPT; a4 += 4) {
        const f32x4 pa = *reinterpret_cast<const f32x4*>(Pt + p * PS + QPT * qg + a4);
        o[a4] += pa.x * vv;
        o[a4 + 1] += pa.y * vv;
        o[a4 + 2] += pa.z * vv;
        o[a4 + 3] += pa.w * vv;
      }
    }
  }
  if (kj == 0) {
    ls[2 * qi] = l[0];
    ls[2 * qi + 1] = l[1];
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < QPT; ++a) {
    const int v = QPT * qg + a, r = v / G, j = v % G;
    if (r < nrows)
      *reinterpret_cast<f32x4*>(o_out + (size_t)(t0 + r) * ldo + (g * G + j) * D + 4 * dg) = o[a] * (1.0f / ls[v]);
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
                             const float* cos_t, const float* sin_t, int nq, int nkv, float* Kc, float* Vc,
                             int max_pos, const DevState* st, int S, int cmin, float* part, float* o_out) {
  const float scale = 1.0f / sqrtf((float)D);
  const dim3 grid(nkv, S);
#define QD_ATTN_DECODE(G_)                                                                                          \
  hipLaunchKernelGGL(k_attn_decode<G_>, grid, dim3(256), 0, s, qkv, qn, kn, eps, cos_t, sin_t, Kc, Vc, max_pos, st, \
                     S, cmin, scale, part)
  switch (nq / nkv) {
    case 1: QD_ATTN_DECODE(1); break;
    case 2: QD_ATTN_DECODE(2); break;
    case 4: QD_ATTN_DECODE(4); break;
    case 8: QD_ATTN_DECODE(8); break;
    default: return;  // rejected by the host before any launch
  }
#undef QD_ATTN_DECODE
  hipLaunchKernelGGL(k_attn_merge_decode, dim3(nq, D / 32), dim3(256), 0, s, part, S, cmin, st, o_out);
}

void launch_attention_prefill(hipStream_t s, const float* q, int T, int nq, int nkv, const float* Kc, const float* Vc,
                              int max_pos, const DevState* st, float* o_out, int ldo, int ncu) {
  const float scale = 1.0f / sqrtf((float)D);
  const int G = nq / nkv;
  // 64 query vectors per block, or 32 when that leaves the GPU under two blocks per CU
  const bool small = (size_t)nkv * ((T + 64 / G - 1) / (64 / G)) < (size_t)2 * ncu;
#define QD_ATTN_PREFILL(G_, QV_)                                                                                    \
  hipLaunchKernelGGL((k_attn_prefill<G_, QV_>), dim3(nkv, (T + QV_ / G_ - 1) / (QV_ / G_)), dim3(256), 0, s, q, T, nq, \
                     Kc, Vc, max_pos, st, scale, o_out, ldo)
  switch (G * (small ? -1 : 1)) {
    case 1: QD_ATTN_PREFILL(1, 64); break;
    case 2: QD_ATTN_PREFILL(2, 64); break;
    case 4: QD_ATTN_PREFILL(4, 64); break;
    case 8: QD_ATTN_PREFILL(8, 64); break;
    case -1: QD_ATTN_PREFILL(1, 32); break;
    case -2: QD_ATTN_PREFILL(2, 32); break;
    case -4: QD_ATTN_PREFILL(4, 32); break;
    case -8: QD_ATTN_PREFILL(8, 32); break;
    default: break;  // rejected by the host before any launch
  }
#undef QD_ATTN_PREFILL
}
