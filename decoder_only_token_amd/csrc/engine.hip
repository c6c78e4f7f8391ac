// Engine and C ABI of libqd (declared in include/qd.h).
//
// One handle = one model on one GPU: engine-owned weights (bf16, or int4
// group-128 codes + fp16 scales), an f32 KV cache laid out
// [layer][kv_head][position][head_dim] (head-major, so a kv head's rows are
// contiguous for the attention scan), host-baked f32 RoPE tables, workspaces
// and the device-resident step state {pos, token, step}.  Every step is
// enqueued on the caller's stream; a decode step is one replay of a captured
// hipGraph that reads pos/token from device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/qd.h"
#include "kernels.h"
#include "persist.h"

namespace {

constexpr int kDecodeMinSplit = 16;  // shortest split of the decode attention
// batches of at most this many rows at positions from kRowAttnMinPos on run
// the split form of the batch attention (its positions cut as the decode
// attention cuts them) instead of the plain one (which spreads a batch over
// its query rows, few here, not over the positions)
constexpr int kRowAttnMaxRows = 16;
constexpr int kRowAttnMinPos = 512;
constexpr int kMaxStepsPerLaunch = 64;  // decode steps in one persistent launch (8-bit step tags, 200 ms waits)
constexpr int kGemmMinRows = 16;  // prefills of at least this many rows use the matrix-core projections

struct Layer {
  uint16_t* wqkv = nullptr;  // [(nq + 2 nkv) d, H]
  float* bqkv = nullptr;     // [(nq + 2 nkv) d] or null
  float* attn_norm = nullptr;
  float* mlp_norm = nullptr;
  float* q_norm = nullptr;
  float* k_norm = nullptr;
  uint16_t* wo = nullptr;  // [H, nq d]
  uint16_t* wg = nullptr;  // [I, H]
  uint16_t* wu = nullptr;  // [I, H]
  uint16_t* wd = nullptr;  // [H, I]
  // int4 group-128 format: codes [rows][in / 2] and fp16 scales [rows][in / 128]
  // of the same five matrices (the bf16 pointers above stay null)
  uint8_t *cqkv = nullptr, *co = nullptr, *cg = nullptr, *cu = nullptr, *cd = nullptr;
  uint16_t *sqkv = nullptr, *so = nullptr, *sg = nullptr, *su = nullptr, *sd = nullptr;
  // Q8_0 format: int8 codes [rows][in] of the five matrices; their fp16 scales
  // [rows][in / 32] use the s* pointers above
  int8_t *qqkv = nullptr, *qo = nullptr, *qg = nullptr, *qu = nullptr, *qd = nullptr;
};

// Adapter of one layer: stacked down matrices [A_q; A_v] [2 r, H] and the up
// matrices B_q [nq d, r], B_v [nkv d, r] (bf16, r = the installed rank).
struct LoraLayer {
  uint16_t* a = nullptr;
  uint16_t* bq = nullptr;
  uint16_t* bv = nullptr;
};

// Keeps the persistent step's abandon flag err[0] as a sticky count err[1] of
// the cache episodes in which a step was abandoned, then clears the flag
// (stream-ordered: no host synchronisation).
__global__ void k_fold_err(uint32_t* err) {
  if (threadIdx.x == 0 && err[0] != 0) {
    err[1] += 1;
    err[0] = 0;
  }
}

__global__ void k_widen_bf16(const uint16_t* __restrict__ src, float* __restrict__ dst, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i < n) dst[i] = __uint_as_float(((uint32_t)src[i]) << 16);
}

}  // namespace

struct qd_handle {
  qd_config cfg{};
  hipStream_t stream = nullptr;
  bool own_stream = false;
  int device = 0;
  std::string err;
  bool weights = false;
  int32_t pos = 0;        // host mirror of DevState::pos
  bool have_token = false;
  std::vector<void*> allocs;

  uint16_t* embed = nullptr;
  float* final_norm = nullptr;
  std::vector<Layer> layers;
  std::vector<LoraLayer> lora;  // sized for lora_rank_max
  int lora_rank = 0;            // 0: no adapter installed
  float lora_scale = 0.f;       // alpha / rank
  float* lu = nullptr;          // [rows][2 lora_rank_max] down products

  float* Kc = nullptr;  // [L][nkv][max_pos][d] f32, or bf16 (kv_format QD_KV_BF16) in the same allocation
  float* Vc = nullptr;
  float* rope_cos = nullptr;  // [max_pos][d/2]
  float* rope_sin = nullptr;

  // workspaces (rows = max_prefill)
  float* x = nullptr;    // [rows][H]
  float* qkv = nullptr;  // [rows][(nq + 2 nkv) d]
  float* q = nullptr;    // [rows][nq][d]
  float* o = nullptr;    // [rows][nq d]
  float* act = nullptr;  // [rows][I]
  uint16_t* xh = nullptr;  // [rows][max(H, nq d, I)] bf16 halves of a projection input
  uint16_t* xl = nullptr;
  uint16_t* xh2 = nullptr;  // [rows][I]: the down projection's input halves (written by gate/up)
  uint16_t* xl2 = nullptr;
  float* gws = nullptr;  // split-K workspace of the batched projections
  size_t gws_floats = 0;
  int ncu = 0;
  float* part = nullptr; // attention partials
  size_t part_floats = 0;
  int dec_splits = 1;    // splits of the decode attention
  float* logits = nullptr;  // [V]
  float* pval = nullptr;
  int32_t* pidx = nullptr;
  // speculative verification: logits [QD_VERIFY_MAX][V], argmax partials
  // [QD_VERIFY_MAX][lmhead_blocks(V)], choices [QD_VERIFY_MAX]
  float* vlogits = nullptr;
  float* vpval = nullptr;
  int32_t* vpidx = nullptr;
  int32_t* vchoice = nullptr;
  float* spv = nullptr;      // sampling: per-slice sorted top-k lists
  int32_t* spi = nullptr;
  int32_t* tokens_dev = nullptr;  // [max_prefill]
  int32_t* tokens_pinned = nullptr;
  DevState* st = nullptr;

  hipGraphExec_t decode_exec = nullptr;
  hipGraph_t decode_graph = nullptr;
  // speculative verification of m rows, captured per [attention mode][m]
  // (mode 1: the split-K decode attention once per row, chosen by position)
  hipGraphExec_t verify_exec[2][QD_VERIFY_MAX + 1] = {};
  hipGraph_t verify_graph[2][QD_VERIFY_MAX + 1] = {};

  // persistent single-kernel decode step
  bool persistent = false;
  int grid = 0;   // one workgroup per CU
  int hseg = 0;   // hidden / 512
  uint32_t seq = 0;
  PersistConst* pconst = nullptr;  // device copy
  LayerPtrs* layer_ptrs = nullptr; // device array [L]
  uint64_t *X0 = nullptr, *X1 = nullptr, *QKVx = nullptr, *PART = nullptr, *Ox = nullptr, *ACT = nullptr;
  uint64_t* AM = nullptr;
  uint64_t* TOK = nullptr;  // the persistent step's token word (multi-step launches)
  uint32_t* err_dev = nullptr;
  bool failed = false;  // a decode step was abandoned; needs qd_reset_kv
  PersistConst pc_host{};
  uint64_t* trace = nullptr;
  bool trace_on = false;
  bool traced_step = false;

  bool capture_on = false;
  float* cap = nullptr;  // [(L + 1)][rows][H] + [H] + [V]
  int32_t cap_rows = 0;  // rows of the last captured prefill (0 = none)

  int set_err(int code, const std::string& m) {
    err = m;
    return code;
  }
};

namespace {

#define HIP_TRY(h, call)                                                                   \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return (h)->set_err(QD_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_));    \
  } while (0)

template <typename T>
int dev_alloc(qd_handle* h, T** p, size_t n) {
  void* v = nullptr;
  // 1 KiB of tail padding: a kernel may read (and ignore) up to one 512-value
  // bf16 segment past the last row of a matrix
  hipError_t e = hipMalloc(&v, n * sizeof(T) + 1024);
  if (e != hipSuccess) return h->set_err(QD_E_OOM, std::string("hipMalloc: ") + hipGetErrorString(e));
  h->allocs.push_back(v);
  *p = static_cast<T*>(v);
  return QD_OK;
}

int qkv_rows(const qd_config& c) { return (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; }

int gemv_t_tile(int K) {
  int t = (16384 - 64) / K;  // keep the staged input (plus the reduction slots) within 64 KiB of LDS
  if (t > GEMV_MAX_T) t = GEMV_MAX_T;
  if (t < 1) t = 1;
  return t;
}

int validate_config(const qd_config* c, std::string& why) {
  if (!c) { why = "config is NULL"; return QD_E_ARG; }
  if (c->struct_size != sizeof(qd_config)) { why = "qd_config.struct_size does not match this library"; return QD_E_ABI; }
  if (c->abi_version != QD_ABI_VERSION) { why = "qd_config.abi_version does not match this library"; return QD_E_ABI; }
  if (c->n_layers < 1 || c->hidden < 256 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->intermediate < 8 ||
      c->vocab < 1) { why = "non-positive or too small model dimension"; return QD_E_ARG; }
  if (c->head_dim != 128) { why = "head_dim must be 128"; return QD_E_ARG; }
  if (c->n_q_heads % c->n_kv_heads) { why = "n_q_heads must be a multiple of n_kv_heads"; return QD_E_ARG; }
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) { why = "n_q_heads / n_kv_heads must be 1, 2, 4 or 8"; return QD_E_ARG; }
  if (c->hidden % 512 || (c->n_q_heads * c->head_dim) % 512) { why = "hidden and n_q_heads*head_dim must be multiples of 512"; return QD_E_ARG; }
  if (c->intermediate % 128) { why = "intermediate must be a multiple of 128"; return QD_E_ARG; }
  if (c->max_prefill >= kGemmMinRows && (!gemm_supported(c->hidden) || !gemm_supported(c->intermediate) ||
                                         !gemm_supported(c->n_q_heads * c->head_dim))) {
    why = "hidden, intermediate and n_q_heads*head_dim must be multiples of 64 for batched prefill";
    return QD_E_ARG;
  }
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) { why = "rope_theta must be > 0 and rms_eps >= 0"; return QD_E_ARG; }
  if (c->tie_embeddings != 1) { why = "only tied embeddings are supported (tie_embeddings must be 1)"; return QD_E_ARG; }
  if (c->weight_format != QD_W_BF16 && c->weight_format != QD_W_INT4_G128 && c->weight_format != QD_W_Q8_0) {
    why = "unknown weight_format";
    return QD_E_ARG;
  }
  if (c->weight_format == QD_W_Q8_0 && c->decode_path != QD_DECODE_GRAPH) {
    why = "Q8_0 weights need decode_path QD_DECODE_GRAPH";
    return QD_E_ARG;
  }
  if (c->max_pos < 1 || c->max_pos > (1 << 20)) { why = "max_pos out of range"; return QD_E_ARG; }
  if (c->max_prefill < 1 || c->max_prefill > c->max_pos) { why = "max_prefill must be in [1, max_pos]"; return QD_E_ARG; }
  if (c->lora_rank_max < 0 || c->lora_rank_max > 64) { why = "lora_rank_max must be in [0, 64]"; return QD_E_ARG; }
  if (c->decode_path != QD_DECODE_PERSISTENT && c->decode_path != QD_DECODE_GRAPH) { why = "unknown decode_path"; return QD_E_ARG; }
  if (c->kv_format != QD_KV_F32 && c->kv_format != QD_KV_BF16) { why = "unknown kv_format"; return QD_E_ARG; }
  if (c->kv_format == QD_KV_BF16 && c->decode_path != QD_DECODE_GRAPH) {
    why = "a bf16 KV cache needs decode_path QD_DECODE_GRAPH";
    return QD_E_ARG;
  }
  if (c->decode_path == QD_DECODE_PERSISTENT) {
    // handshake tags carry the layer in 8 bits; 255 marks the argmax words and the unset value pairs
    if (c->n_layers > 254) { why = "the persistent decode step supports at most 254 layers"; return QD_E_ARG; }
    if (c->lora_rank_max != 0) {
      // the LoRA-down CU holds [A_q; A_v] in the 24 registers slots per lane it
      // loads ahead (rows over 8 waves, 512 columns a slot), and an attention
      // item stages its heads' B rows (bf16) in the 2 x 11264 floats of the
      // phase-input slots
      const int G = c->n_kv_heads > 0 ? c->n_q_heads / c->n_kv_heads : 0;
      if ((2 * c->lora_rank_max + 7) / 8 * ((c->hidden + 511) / 512) > 24 ||
          (size_t)(G + 1) * c->head_dim * c->lora_rank_max * 2 > 2 * 11264 * 4) {
        why = "lora_rank_max too large for the persistent decode step (ceil(r / 4) * hidden / 512 must be <= 24)";
        return QD_E_ARG;
      }
    }
    if (c->hidden != 1024 && c->hidden != 2048) { why = "the persistent decode step needs hidden 1024 or 2048"; return QD_E_ARG; }
    if (c->intermediate > 11264 || c->n_q_heads * c->head_dim > 11264) { why = "model too wide for the persistent decode step"; return QD_E_ARG; }
  }
  return QD_OK;
}

// Split-K workspace for the batched projections: the largest need over the
// prefill lengths that use them and the four products of a layer.
int alloc_gemm_workspace(qd_handle* h) {
  const qd_config& c = h->cfg;
  if (c.max_prefill < kGemmMinRows) return QD_OK;
  size_t need = 0;
  const int NQKV = qkv_rows(c);
  // the need s(T) * T * N peaks at the end of each row-tile count (64 or 128 rows)
  for (int T = std::min(64, c.max_prefill); T <= c.max_prefill; T = T < c.max_prefill ? std::min(T + 64, c.max_prefill) : T + 1) {
    need = std::max(need, gemm_workspace_floats(T, c.hidden, NQKV, h->ncu));
    need = std::max(need, gemm_workspace_floats(T, c.n_q_heads * c.head_dim, c.hidden, h->ncu));
    need = std::max(need, gemm_workspace_floats(T, c.hidden, c.intermediate, h->ncu));
    need = std::max(need, gemm_workspace_floats(T, c.intermediate, c.hidden, h->ncu));
    if (c.lora_rank_max) need = std::max(need, gemm_workspace_floats(T, c.hidden, 2 * c.lora_rank_max, h->ncu));
  }
  h->gws_floats = need;
  return need ? dev_alloc(h, &h->gws, need) : QD_OK;
}

int build_rope_tables(qd_handle* h) {
  const qd_config& c = h->cfg;
  const int half = c.head_dim / 2;
  std::vector<float> cs((size_t)c.max_pos * half), sn((size_t)c.max_pos * half);
  for (int j = 0; j < half; ++j) {
    const double inv = std::pow((double)c.rope_theta, -2.0 * j / c.head_dim);
    for (int p = 0; p < c.max_pos; ++p) {
      const double a = (double)p * inv;
      cs[(size_t)p * half + j] = (float)std::cos(a);
      sn[(size_t)p * half + j] = (float)std::sin(a);
    }
  }
  HIP_TRY(h, hipMemcpy(h->rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
  HIP_TRY(h, hipMemcpy(h->rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
  return QD_OK;
}

void drop_decode_graph(qd_handle* h) {
  if (h->decode_exec) (void)hipGraphExecDestroy(h->decode_exec);
  if (h->decode_graph) (void)hipGraphDestroy(h->decode_graph);
  h->decode_exec = nullptr;
  h->decode_graph = nullptr;
  for (int a = 0; a < 2; ++a)
    for (int m = 0; m <= QD_VERIFY_MAX; ++m) {
      if (h->verify_exec[a][m]) (void)hipGraphExecDestroy(h->verify_exec[a][m]);
      if (h->verify_graph[a][m]) (void)hipGraphDestroy(h->verify_graph[a][m]);
      h->verify_exec[a][m] = nullptr;
      h->verify_graph[a][m] = nullptr;
    }
}

void free_all(qd_handle* h) {
  drop_decode_graph(h);
  for (void* p : h->allocs) (void)hipFree(p);
  h->allocs.clear();
  if (h->tokens_pinned) (void)hipHostFree(h->tokens_pinned);
  h->tokens_pinned = nullptr;
  if (h->own_stream && h->stream) (void)hipStreamDestroy(h->stream);
  h->stream = nullptr;
}

void enqueue_layers_gemm(qd_handle* h, int T, bool capture);
void enqueue_layers_gemv(qd_handle* h, int T, bool capture);

// Enqueue the whole forward for T new rows whose ids are at `tok` (device),
// at positions st->pos .. st->pos + T - 1, and choose the next token from the
// last row.  Captures are written only when `capture` is set.
void enqueue_forward(qd_handle* h, int T, const int32_t* tok, bool capture) {
  const qd_config& c = h->cfg;
  hipStream_t s = h->stream;
  const int H = c.hidden;
  launch_embed(s, h->embed, tok, T, H, h->x);
  if (capture) (void)hipMemcpyAsync(h->cap, h->x, (size_t)T * H * 4, hipMemcpyDeviceToDevice, s);
  if (T >= kGemmMinRows && c.weight_format != QD_W_Q8_0) {  // (Q8_0: the GEMVs on row tiles)
    enqueue_layers_gemm(h, T, capture);
  } else {
    enqueue_layers_gemv(h, T, capture);
  }
  float* xf_cap = capture ? h->cap + (size_t)(c.n_layers + 1) * c.max_prefill * H : nullptr;
  const int nparts = launch_lmhead_bf16(s, h->embed, c.vocab, H, h->x + (size_t)(T - 1) * H, h->final_norm,
                                       c.rms_eps, h->logits, h->pval, h->pidx, xf_cap);
  launch_argmax_final(s, h->pval, h->pidx, nparts, h->st, T, nullptr);
  if (capture)
    (void)hipMemcpyAsync(xf_cap + H, h->logits, (size_t)c.vocab * 4, hipMemcpyDeviceToDevice, s);
}

// Attention for T new rows (shared by both projection paths).
// Layer l's block of a KV cache (elements of 4 or 2 bytes).
void* kv_layer(qd_handle* h, float* base, int l) {
  const qd_config& c = h->cfg;
  const size_t layer_kv = (size_t)c.n_kv_heads * c.max_pos * c.head_dim;
  return reinterpret_cast<char*>(base) + l * layer_kv * (c.kv_format == QD_KV_BF16 ? 2 : 4);
}

// hilo_o: the batch attention also writes the bf16 halves of its output into
// xh / xl (the o_proj input of the matrix-core projections); returns whether it did.
bool enqueue_attention(qd_handle* h, int l, int T, bool hilo_o = false) {
  const qd_config& c = h->cfg;
  hipStream_t s = h->stream;
  const int d = c.head_dim, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const int kv16 = c.kv_format == QD_KV_BF16;
  const Layer& L = h->layers[l];
  LoraRows lr;  // a batch's adapter up products: added by the QK-norm / RoPE pass
  if (h->lora_rank) {
    lr.u = h->lu;
    lr.ldu = 2 * h->lora_rank;
    lr.bq = h->lora[l].bq;
    lr.bv = h->lora[l].bv;
    lr.r = h->lora_rank;
    lr.scale = h->lora_scale;
  }
  if (T == 1) {  // QK-norm, RoPE, the adapter's up products and the cache write happen inside the decode attention
    const bool lo = h->lora_rank > 0;
    launch_attention_decode(s, h->qkv, L.q_norm, L.k_norm, c.rms_eps, h->rope_cos, h->rope_sin, nq, nkv,
                            kv_layer(h, h->Kc, l), kv_layer(h, h->Vc, l), kv16, c.max_pos, h->st, h->dec_splits,
                            kDecodeMinSplit, h->part, h->o, lo ? h->lu : nullptr, lo ? h->lora[l].bq : nullptr,
                            lo ? h->lora[l].bv : nullptr, h->lora_rank, h->lora_scale);
  } else if (T <= kRowAttnMaxRows && h->pos >= kRowAttnMinPos) {
    // a few rows at a long context (speculative verification, short prefills):
    // the adapter, QK-norm, RoPE and the cache rows of all of them, then one
    // split-K pass over the positions for every row at once (the decode
    // attention's splits, so the batch is spread over the CUs) and the rows'
    // merges
    launch_qk_rope_kv(s, h->qkv, qkv_rows(c), T, nq, nkv, d, L.q_norm, L.k_norm, c.rms_eps, h->rope_cos, h->rope_sin,
                      h->st, h->q, kv_layer(h, h->Kc, l), kv_layer(h, h->Vc, l), c.max_pos, kv16, lr);
    launch_attention_rows_split(s, h->q, T, nq, nkv, kv_layer(h, h->Kc, l), kv_layer(h, h->Vc, l), kv16, c.max_pos,
                                h->st, h->dec_splits, kDecodeMinSplit, h->part, h->o);
  } else {
    launch_qk_rope_kv(s, h->qkv, qkv_rows(c), T, nq, nkv, d, L.q_norm, L.k_norm, c.rms_eps, h->rope_cos, h->rope_sin,
                      h->st, h->q, kv_layer(h, h->Kc, l), kv_layer(h, h->Vc, l), c.max_pos, kv16, lr);
    launch_attention_prefill(s, h->q, T, nq, nkv, kv_layer(h, h->Kc, l), kv_layer(h, h->Vc, l), kv16, c.max_pos, h->st,
                             h->o, nq * d, h->ncu, h->part, kDecodeMinSplit, hilo_o ? h->xh : nullptr,
                             hilo_o ? h->xl : nullptr);
    return hilo_o;
  }
  return false;
}

// Layers with the matrix-core projections (T >= kGemmMinRows).
void enqueue_layers_gemm(qd_handle* h, int T, bool capture) {
  const qd_config& c = h->cfg;
  const bool q4 = c.weight_format == QD_W_INT4_G128;
  hipStream_t s = h->stream;
  const int H = c.hidden, d = c.head_dim, nq = c.n_q_heads, I = c.intermediate;
  const int NQKV = qkv_rows(c);
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& L = h->layers[l];
    launch_split_rows(s, h->x, H, T, H, L.attn_norm, c.rms_eps, h->xh, h->xl);
    if (q4)
      launch_gemm_q4(s, GEMM_STORE, h->xh, h->xl, T, H, L.cqkv, L.sqkv, nullptr, nullptr, NQKV, L.bqkv, h->qkv, NQKV,
                     h->gws, h->gws_floats, h->ncu);
    else
      launch_gemm_hilo(s, GEMM_STORE, h->xh, h->xl, T, H, L.wqkv, nullptr, NQKV, L.bqkv, h->qkv, NQKV, h->gws,
                       h->gws_floats, h->ncu);
    if (h->lora_rank) {  // the down products (the normed input halves are still in xh / xl)
      const int r2 = 2 * h->lora_rank;
      launch_gemm_hilo(s, GEMM_STORE, h->xh, h->xl, T, H, h->lora[l].a, nullptr, r2, nullptr, h->lu, r2, h->gws,
                       h->gws_floats, h->ncu);
    }
    if (!enqueue_attention(h, l, T, true))  // (else the attention wrote the o_proj input halves)
      launch_split_rows(s, h->o, nq * d, T, nq * d, nullptr, 0.f, h->xh, h->xl);
    if (q4)
      launch_gemm_q4(s, GEMM_ADD, h->xh, h->xl, T, nq * d, L.co, L.so, nullptr, nullptr, H, nullptr, h->x, H, h->gws,
                     h->gws_floats, h->ncu);
    else
      launch_gemm_hilo(s, GEMM_ADD, h->xh, h->xl, T, nq * d, L.wo, nullptr, H, nullptr, h->x, H, h->gws,
                       h->gws_floats, h->ncu);
    launch_split_rows(s, h->x, H, T, H, L.mlp_norm, c.rms_eps, h->xh, h->xl);
    // gate | up writes SiLU(gate) * up and its bf16 halves (the down input)
    if (q4)
      launch_gemm_q4(s, GEMM_GATEUP, h->xh, h->xl, T, H, L.cg, L.sg, L.cu, L.su, I, nullptr, h->act, I, h->gws,
                     h->gws_floats, h->ncu, h->xh2, h->xl2);
    else
      launch_gemm_hilo(s, GEMM_GATEUP, h->xh, h->xl, T, H, L.wg, L.wu, I, nullptr, h->act, I, h->gws, h->gws_floats,
                       h->ncu, h->xh2, h->xl2);
    if (q4)
      launch_gemm_q4(s, GEMM_ADD, h->xh2, h->xl2, T, I, L.cd, L.sd, nullptr, nullptr, H, nullptr, h->x, H, h->gws,
                     h->gws_floats, h->ncu);
    else
      launch_gemm_hilo(s, GEMM_ADD, h->xh2, h->xl2, T, I, L.wd, nullptr, H, nullptr, h->x, H, h->gws, h->gws_floats,
                       h->ncu);
    if (capture)
      (void)hipMemcpyAsync(h->cap + (size_t)(l + 1) * c.max_prefill * H, h->x, (size_t)T * H * 4,
                           hipMemcpyDeviceToDevice, s);
  }
}

// Layers with the T-row GEMV projections (decode and short prefills).
void enqueue_layers_gemv(qd_handle* h, int T, bool capture) {
  const qd_config& c = h->cfg;
  hipStream_t s = h->stream;
  const int H = c.hidden, d = c.head_dim, nq = c.n_q_heads, I = c.intermediate;
  const int NQKV = qkv_rows(c);
  const bool q4 = c.weight_format == QD_W_INT4_G128, q8 = c.weight_format == QD_W_Q8_0;
  auto tile = [&](int K) { return q4 ? q4_gemv_t_tile(K) : q8 ? q8_gemv_t_tile(K) : gemv_t_tile(K); };
  // int4 o_proj, gate/up and down: row tiles of the matrix-core forms where
  // they cover the width (one row: the single-row form)
  auto tile4 = [&](int K, bool gu) { return q4 && q4mr_rows(K, gu) ? q4mr_rows(K, gu) : tile(K); };
  // int4 q|k|v of a batch on the matrix cores (the adapter's down products
  // then run as their own bf16 GEMV); of a single row, the VALU GEMV with the
  // down products riding along as bf16 rows
  const bool qkv_mr = q4 && T > 1 && q4mr_rows(H, false);
  for (int l = 0; l < c.n_layers; ++l) {
    const Layer& L = h->layers[l];
    for (int t0 = 0, tt = qkv_mr ? q4mr_rows(H, false) : tile(H); t0 < T; t0 += tt) {
      const int tn = std::min(tt, T - t0);
      const bool xr = h->lora_rank && !qkv_mr;
      if (qkv_mr && tn > 1 &&
          q4mr_gemv(s, L.cqkv, L.sqkv, NQKV, H, h->x + (size_t)t0 * H, H, tn, L.attn_norm, c.rms_eps, L.bqkv,
                    h->qkv + (size_t)t0 * NQKV, NQKV, 0)) {
      } else if (q4)
        launch_gemv_q4(s, L.cqkv, L.sqkv, NQKV, H, h->x + (size_t)t0 * H, H, tn, L.attn_norm, c.rms_eps, L.bqkv,
                       h->qkv + (size_t)t0 * NQKV, NQKV, 0, h->ncu, xr ? h->lora[l].a : nullptr, xr ? 2 * h->lora_rank : 0,
                       h->lu + (size_t)t0 * 2 * h->lora_rank, 2 * h->lora_rank);
      else if (q8)
        launch_gemv_q8(s, L.qqkv, L.sqkv, NQKV, H, h->x + (size_t)t0 * H, H, tn, L.attn_norm, c.rms_eps, L.bqkv,
                       h->qkv + (size_t)t0 * NQKV, NQKV, 0, h->ncu);
      else
        launch_gemv_bf16(s, L.wqkv, NQKV, H, h->x + (size_t)t0 * H, H, tn, L.attn_norm, c.rms_eps, L.bqkv,
                         h->qkv + (size_t)t0 * NQKV, NQKV, 0, h->ncu);
    }
    if (h->lora_rank) {
      const int r2 = 2 * h->lora_rank;
      const bool own = qkv_mr && launch_lora_down_rows(s, h->lora[l].a, r2, H, h->x, H, T, L.attn_norm, c.rms_eps,
                                                       h->lu, r2);
      for (int t0 = 0, tt = gemv_t_tile(H); t0 < T && (!q4 || qkv_mr) && !own; t0 += tt) {  // (else inside the q|k|v GEMV)
        const int tn = std::min(tt, T - t0);
        launch_gemv_bf16(s, h->lora[l].a, r2, H, h->x + (size_t)t0 * H, H, tn, L.attn_norm, c.rms_eps, nullptr,
                         h->lu + (size_t)t0 * r2, r2, 0, h->ncu);
      }
    }
    enqueue_attention(h, l, T);
    for (int t0 = 0, tt = tile4(nq * d, false); t0 < T; t0 += tt) {
      const int tn = std::min(tt, T - t0);
      if (q4 && tn == 1 &&
          q4m_gemv(s, L.co, L.so, H, nq * d, h->o + (size_t)t0 * nq * d, nullptr, 0.f, nullptr, h->x + (size_t)t0 * H, 1)) {
      } else if (q4 && tn > 1 &&
                 q4mr_gemv(s, L.co, L.so, H, nq * d, h->o + (size_t)t0 * nq * d, nq * d, tn, nullptr, 0.f, nullptr,
                           h->x + (size_t)t0 * H, H, 1)) {
      } else if (q4)
        launch_gemv_q4(s, L.co, L.so, H, nq * d, h->o + (size_t)t0 * nq * d, nq * d, tn, nullptr, 0.f, nullptr,
                       h->x + (size_t)t0 * H, H, 1, h->ncu);
      else if (q8)
        launch_gemv_q8(s, L.qo, L.so, H, nq * d, h->o + (size_t)t0 * nq * d, nq * d, tn, nullptr, 0.f, nullptr,
                       h->x + (size_t)t0 * H, H, 1, h->ncu);
      else
        launch_gemv_bf16(s, L.wo, H, nq * d, h->o + (size_t)t0 * nq * d, nq * d, tn, nullptr, 0.f, nullptr,
                         h->x + (size_t)t0 * H, H, 1, h->ncu);
    }
    for (int t0 = 0, tt = tile4(H, true); t0 < T; t0 += tt) {
      const int tn = std::min(tt, T - t0);
      if (q4 && tn > 1 &&
          q4mr_gateup(s, L.cg, L.sg, L.cu, L.su, I, H, h->x + (size_t)t0 * H, H, tn, L.mlp_norm, c.rms_eps,
                      h->act + (size_t)t0 * I, I)) {
      } else if (q4 && tn == 1 &&
          q4m_gateup(s, L.cg, L.sg, L.cu, L.su, I, H, h->x + (size_t)t0 * H, L.mlp_norm, c.rms_eps, h->act + (size_t)t0 * I)) {
      } else if (q4)
        launch_gemv_gateup_q4(s, L.cg, L.sg, L.cu, L.su, I, H, h->x + (size_t)t0 * H, H, tn, L.mlp_norm, c.rms_eps,
                              h->act + (size_t)t0 * I, I, h->ncu);
      else if (q8)
        launch_gemv_gateup_q8(s, L.qg, L.sg, L.qu, L.su, I, H, h->x + (size_t)t0 * H, H, tn, L.mlp_norm, c.rms_eps,
                              h->act + (size_t)t0 * I, I, h->ncu);
      else
        launch_gemv_gateup_bf16(s, L.wg, L.wu, I, H, h->x + (size_t)t0 * H, H, tn, L.mlp_norm, c.rms_eps,
                                h->act + (size_t)t0 * I, I, h->ncu);
    }
    for (int t0 = 0, tt = tile4(I, false); t0 < T; t0 += tt) {
      const int tn = std::min(tt, T - t0);
      if (q4 && tn == 1 &&
          q4m_gemv(s, L.cd, L.sd, H, I, h->act + (size_t)t0 * I, nullptr, 0.f, nullptr, h->x + (size_t)t0 * H, 1)) {
      } else if (q4 && tn > 1 &&
                 q4mr_gemv(s, L.cd, L.sd, H, I, h->act + (size_t)t0 * I, I, tn, nullptr, 0.f, nullptr,
                           h->x + (size_t)t0 * H, H, 1)) {
      } else if (q4)
        launch_gemv_q4(s, L.cd, L.sd, H, I, h->act + (size_t)t0 * I, I, tn, nullptr, 0.f, nullptr,
                       h->x + (size_t)t0 * H, H, 1, h->ncu);
      else if (q8)
        launch_gemv_q8(s, L.qd, L.sd, H, I, h->act + (size_t)t0 * I, I, tn, nullptr, 0.f, nullptr,
                       h->x + (size_t)t0 * H, H, 1, h->ncu);
      else
        launch_gemv_bf16(s, L.wd, H, I, h->act + (size_t)t0 * I, I, tn, nullptr, 0.f, nullptr,
                         h->x + (size_t)t0 * H, H, 1, h->ncu);
    }
    if (capture)
      (void)hipMemcpyAsync(h->cap + (size_t)(l + 1) * c.max_prefill * H, h->x, (size_t)T * H * 4, hipMemcpyDeviceToDevice,
                     s);
  }
}

int copy_outputs(qd_handle* h, float* logits_dev, int32_t* token_dev) {
  if (logits_dev)
    HIP_TRY(h, hipMemcpyAsync(logits_dev, h->logits, (size_t)h->cfg.vocab * 4, hipMemcpyDeviceToDevice, h->stream));
  if (token_dev)
    HIP_TRY(h, hipMemcpyAsync(token_dev, &h->st->token, 4, hipMemcpyDeviceToDevice, h->stream));
  return QD_OK;
}

int check_sampling(qd_handle* h, const qd_sampling* sp) {
  if (!sp) return QD_OK;
  if (sp->struct_size != sizeof(qd_sampling)) return h->set_err(QD_E_ABI, "qd_sampling.struct_size mismatch");
  if (!(sp->temperature <= 0.f) && !(sp->temperature > 0.f && std::isfinite(sp->temperature)))
    return h->set_err(QD_E_ARG, "temperature must be finite");
  if (sp->temperature <= 0.f) return QD_OK;
  if (sp->top_k < 1 || sp->top_k > 64) return h->set_err(QD_E_ARG, "top_k must be in [1, 64]");
  if (!sample_supported(h->cfg.vocab, sp->top_k)) return h->set_err(QD_E_ARG, "top_k too large for this vocabulary");
  if (!(sp->top_p > 0.f && sp->top_p <= 1.f)) return h->set_err(QD_E_ARG, "top_p must be in (0, 1]");
  return QD_OK;
}

// After the greedy pass has written the logits and counted the token: replace
// its choice by a draw when sampling is asked for (top_k == 1 is greedy).
int maybe_sample(qd_handle* h, const qd_sampling* sp) {
  if (!sp || sp->temperature <= 0.f || sp->top_k == 1) return QD_OK;
  launch_sample(h->stream, h->logits, h->cfg.vocab, sp->top_k, sp->temperature, sp->top_p, sp->seed, h->spv, h->spi,
                h->st, 0, nullptr);
  HIP_TRY(h, hipGetLastError());
  return QD_OK;
}

}  // namespace

extern "C" {

size_t qd_sizeof_config(void) { return sizeof(qd_config); }
size_t qd_sizeof_weights(void) { return sizeof(qd_weights); }
size_t qd_sizeof_sampling(void) { return sizeof(qd_sampling); }
size_t qd_sizeof_lora(void) { return sizeof(qd_lora); }

const char* qd_last_error(const qd_handle* h) { return h ? h->err.c_str() : sample_free_error(); }

// The persistent step's value-pair buffers (16-bit tags) to all ones: a tag
// of layer 255, which no decoder layer uses, so no stale word matches.  A
// null stream fills synchronously.
static int fill_pairs(qd_handle* h, hipStream_t st) {
  const qd_config& c = h->cfg;
  struct { uint64_t* p; size_t words; } bufs[] = {{h->ACT, (size_t)c.intermediate},
                                                  {h->Ox, (size_t)c.n_q_heads * c.head_dim}};
  for (auto& b : bufs) {
    const hipError_t e = st ? hipMemsetAsync(b.p, 0xFF, b.words * 8, st) : hipMemset(b.p, 0xFF, b.words * 8);
    if (e != hipSuccess) return QD_E_HIP;
  }
  return QD_OK;
}

int qd_create(const qd_config* cfg, void* hip_stream, qd_handle** out) {
  if (!out) return QD_E_ARG;
  *out = nullptr;
  std::string why;
  int rc = validate_config(cfg, why);
  if (rc != QD_OK) {
    fprintf(stderr, "qd_create: %s\n", why.c_str());
    return rc;
  }
  qd_handle* h = new qd_handle();
  h->cfg = *cfg;
  const qd_config& c = h->cfg;
  auto fail = [&](int code) {
    fprintf(stderr, "qd_create: %s\n", h->err.c_str());
    free_all(h);
    delete h;
    return code;
  };
  if (hipGetDevice(&h->device) != hipSuccess) return fail(h->set_err(QD_E_HIP, "hipGetDevice failed"));
  if (hipDeviceGetAttribute(&h->ncu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || h->ncu < 1)
    return fail(h->set_err(QD_E_HIP, "cannot query the CU count"));
  if (hip_stream) {
    h->stream = (hipStream_t)hip_stream;
  } else {
    if (hipStreamCreateWithFlags(&h->stream, hipStreamNonBlocking) != hipSuccess)
      return fail(h->set_err(QD_E_HIP, "hipStreamCreate failed"));
    h->own_stream = true;
  }
  const size_t H = c.hidden, d = c.head_dim, I = c.intermediate, rows = c.max_prefill;
  // KV elements as floats: a bf16 cache takes half (rounded up)
  const size_t kv_elems = (size_t)c.n_layers * c.n_kv_heads * c.max_pos * d + 256 * d;
  const size_t kvf = c.kv_format == QD_KV_BF16 ? (kv_elems + 1) / 2 : kv_elems;
  h->dec_splits = attn_decode_splits(c.max_pos, c.n_kv_heads, h->ncu, kDecodeMinSplit);
  // attention partials: a short batch's rows over the decode splits, or a
  // prefill's rows over its splits (batches whose query tiles leave CUs idle)
  size_t part_rows = (size_t)kRowAttnMaxRows * h->dec_splits;
  for (int t = 2; t <= c.max_prefill; ++t)
    part_rows = std::max(part_rows, (size_t)t * attn_prefill_splits(t, c.n_q_heads, c.n_kv_heads, h->ncu));
  h->part_floats = part_rows * c.n_q_heads * (d + 2);
  // the caches carry 256 rows of tail padding: the persistent decode step reads
  // (and ignores) up to 192 positions past the end of a split
  if ((rc = dev_alloc(h, &h->Kc, kvf)) || (rc = dev_alloc(h, &h->Vc, kvf)) ||
      (rc = dev_alloc(h, &h->rope_cos, (size_t)c.max_pos * d / 2)) ||
      (rc = dev_alloc(h, &h->rope_sin, (size_t)c.max_pos * d / 2)) || (rc = dev_alloc(h, &h->x, rows * H)) ||
      (rc = dev_alloc(h, &h->qkv, rows * qkv_rows(c))) || (rc = dev_alloc(h, &h->q, rows * c.n_q_heads * d)) ||
      (rc = dev_alloc(h, &h->o, rows * c.n_q_heads * d)) || (rc = dev_alloc(h, &h->act, rows * I)) ||
      (rc = dev_alloc(h, &h->xh, rows * std::max(std::max(H, (size_t)c.n_q_heads * d), I))) ||
      (rc = dev_alloc(h, &h->xl, rows * std::max(std::max(H, (size_t)c.n_q_heads * d), I))) ||
      (rc = dev_alloc(h, &h->xh2, rows * I)) || (rc = dev_alloc(h, &h->xl2, rows * I)) ||
      (rc = alloc_gemm_workspace(h)) ||
      (rc = dev_alloc(h, &h->part, h->part_floats)) || (rc = dev_alloc(h, &h->logits, (size_t)c.vocab)) ||
      (rc = dev_alloc(h, &h->pval, (size_t)lmhead_blocks(c.vocab))) ||
      (rc = dev_alloc(h, &h->pidx, (size_t)lmhead_blocks(c.vocab))) ||
      (rc = dev_alloc(h, &h->vlogits, (size_t)QD_VERIFY_MAX * c.vocab)) ||
      (rc = dev_alloc(h, &h->vpval, (size_t)QD_VERIFY_MAX * lmhead_blocks(c.vocab))) ||
      (rc = dev_alloc(h, &h->vpidx, (size_t)QD_VERIFY_MAX * lmhead_blocks(c.vocab))) ||
      (rc = dev_alloc(h, &h->vchoice, (size_t)QD_VERIFY_MAX)) ||
      (rc = dev_alloc(h, &h->spv, (size_t)sample_lists(c.vocab) * 64)) ||
      (rc = dev_alloc(h, &h->spi, (size_t)sample_lists(c.vocab) * 64)) ||
      (rc = dev_alloc(h, &h->tokens_dev, rows)) || (rc = dev_alloc(h, &h->st, 1)))
    return fail(rc);
  // caches start as zeros, padding included (rows are read past a split's end
  // and discarded; zeros keep even the discarded values finite)
  if (hipMemset(h->Kc, 0, kvf * sizeof(float)) != hipSuccess ||
      hipMemset(h->Vc, 0, kvf * sizeof(float)) != hipSuccess)
    return fail(h->set_err(QD_E_HIP, "hipMemset failed"));
  if (hipHostMalloc((void**)&h->tokens_pinned, rows * sizeof(int32_t), hipHostMallocDefault) != hipSuccess)
    return fail(h->set_err(QD_E_OOM, "hipHostMalloc failed"));
  if ((rc = build_rope_tables(h))) return fail(rc);
  if (sample_supported(c.vocab, 1) && sample_prepare() != 0)
    return fail(h->set_err(QD_E_HIP, "sampling kernel unavailable"));
  if (c.decode_path == QD_DECODE_PERSISTENT) {
    h->persistent = true;
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess || ncu < 1)
      return fail(h->set_err(QD_E_HIP, "cannot query the CU count"));
    h->grid = ncu > 1024 ? 1024 : ncu;
    if (const char* e = getenv("QD_PERSIST_CUS")) {  // fewer workgroups (diagnostics, tests)
      const int n = atoi(e);
      if (n >= 1 && n < h->grid) h->grid = n;
    }
    h->hseg = c.hidden / 512;
    const int G = c.n_q_heads / c.n_kv_heads;
    const int q4 = c.weight_format == QD_W_INT4_G128;
    if (persist_prepare(G, h->hseg, q4, 0) != 0 || (c.lora_rank_max && persist_prepare(G, h->hseg, q4, 1) != 0))
      return fail(h->set_err(QD_E_HIP, "persistent decode kernel unavailable"));
    {  // the role plan must exist at the shortest and the longest context
      PersistConst shape{};
      shape.q4 = q4;
      shape.H = c.hidden; shape.nq = c.n_q_heads; shape.nkv = c.n_kv_heads; shape.I = c.intermediate;
      shape.nqkv = (int)qkv_rows(c); shape.max_pos = c.max_pos; shape.V = c.vocab;
      shape.lora_r = c.lora_rank_max;  // the plan with the LoRA-down CU, if an adapter may come
      PersistStep st;
      if (c.vocab < h->grid || persist_plan(shape, h->grid, 0, 1, &st) != 0 ||
          persist_plan(shape, h->grid, c.max_pos - 1, 1, &st) != 0)
        return fail(h->set_err(QD_E_ARG, "the model does not fit the CU roles of the persistent decode step"));
    }
    const size_t smax = (size_t)h->grid / c.n_kv_heads;
    if ((rc = dev_alloc(h, &h->X0, H)) || (rc = dev_alloc(h, &h->X1, H)) ||
        (rc = dev_alloc(h, &h->QKVx, (size_t)qkv_rows(c) + 2 * c.lora_rank_max)) ||
        (rc = dev_alloc(h, &h->PART, (size_t)c.n_q_heads * smax * (d + 2))) ||
        (rc = dev_alloc(h, &h->Ox, (size_t)c.n_q_heads * d)) || (rc = dev_alloc(h, &h->ACT, I)) ||
        (rc = dev_alloc(h, &h->AM, (size_t)2 * h->grid)) || (rc = dev_alloc(h, &h->TOK, 1)) ||
        (rc = dev_alloc(h, &h->err_dev, 4)) || (rc = dev_alloc(h, &h->pconst, 1)) ||
        (rc = dev_alloc(h, &h->layer_ptrs, (size_t)c.n_layers)))
      return fail(rc);
    // tags start at 0; every step uses seq >= 1, so stale words never match.
    // The value-pair buffers carry only 16 tag bits (8 of the step): they start
    // as all ones (layer 255, never a decoder layer), and a reset refills them.
    if (hipMemset(h->X0, 0, H * 8) || hipMemset(h->X1, 0, H * 8) || hipMemset(h->QKVx, 0, (qkv_rows(c) + 2 * c.lora_rank_max) * 8) ||
        hipMemset(h->PART, 0, (size_t)c.n_q_heads * smax * (d + 2) * 8) || hipMemset(h->AM, 0, h->grid * 16) || hipMemset(h->TOK, 0, 8) ||
        hipMemset(h->err_dev, 0, 16) || fill_pairs(h, nullptr) != QD_OK)
      return fail(h->set_err(QD_E_HIP, "hipMemset failed"));
  }
  if (hipMemset(h->st, 0, sizeof(DevState)) != hipSuccess) return fail(h->set_err(QD_E_HIP, "hipMemset failed"));
  h->layers.resize(c.n_layers);
  if (c.lora_rank_max) {
    const size_t r = c.lora_rank_max;
    h->lora.resize(c.n_layers);
    if ((rc = dev_alloc(h, &h->lu, rows * 2 * r))) return fail(rc);
    for (auto& A : h->lora)
      if ((rc = dev_alloc(h, &A.a, 2 * r * H)) || (rc = dev_alloc(h, &A.bq, (size_t)c.n_q_heads * d * r)) ||
          (rc = dev_alloc(h, &A.bv, (size_t)c.n_kv_heads * d * r)))
        return fail(rc);
  }
  *out = h;
  return QD_OK;
}

int qd_load_weights(qd_handle* h, const qd_weights* w) {
  if (!h) return QD_E_ARG;
  if (!w) return h->set_err(QD_E_ARG, "weights is NULL");
  if (w->struct_size != sizeof(qd_weights)) return h->set_err(QD_E_ABI, "qd_weights.struct_size mismatch");
  const qd_config& c = h->cfg;
  if (w->lm_head) return h->set_err(QD_E_ARG, "lm_head must be NULL for tied embeddings");
  if (!w->embed || !w->final_norm || !w->attn_norm || !w->mlp_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->w_gate || !w->w_up || !w->w_down)
    return h->set_err(QD_E_ARG, "a required weight array is NULL");
  if (c.qk_norm && (!w->q_norm || !w->k_norm)) return h->set_err(QD_E_ARG, "q_norm/k_norm required");
  if (c.qkv_bias && (!w->bq || !w->bk || !w->bv)) return h->set_err(QD_E_ARG, "bq/bk/bv required");
  for (int l = 0; l < c.n_layers; ++l) {
    if (!w->attn_norm[l] || !w->mlp_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->w_gate[l] ||
        !w->w_up[l] || !w->w_down[l] || (c.qk_norm && (!w->q_norm[l] || !w->k_norm[l])) ||
        (c.qkv_bias && (!w->bq[l] || !w->bk[l] || !w->bv[l])))
      return h->set_err(QD_E_ARG, "NULL pointer in layer " + std::to_string(l));
  }
  const size_t H = c.hidden, d = c.head_dim, I = c.intermediate, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const size_t NQKV = qkv_rows(c), G = nq / nkv;
  hipStream_t s = h->stream;
  int rc;
  auto widen = [&](const void* src, float* dst, size_t n) {
    hipLaunchKernelGGL(k_widen_bf16, dim3((n + 255) / 256), dim3(256), 0, s, (const uint16_t*)src, dst, n);
  };
  const bool q4 = c.weight_format == QD_W_INT4_G128, q8 = c.weight_format == QD_W_Q8_0;
  if (!h->weights) {  // first load: allocate engine-owned weight buffers
    if ((rc = dev_alloc(h, &h->embed, (size_t)c.vocab * H)) || (rc = dev_alloc(h, &h->final_norm, H))) return rc;
    for (auto& L : h->layers) {
      if ((rc = dev_alloc(h, &L.attn_norm, H)) || (rc = dev_alloc(h, &L.mlp_norm, H))) return rc;
      if (q4) {
        if ((rc = dev_alloc(h, &L.cqkv, NQKV * H / 2)) || (rc = dev_alloc(h, &L.sqkv, NQKV * H / 128)) ||
            (rc = dev_alloc(h, &L.co, H * nq * d / 2)) || (rc = dev_alloc(h, &L.so, H * nq * d / 128)) ||
            (rc = dev_alloc(h, &L.cg, 2 * I * H / 2)) || (rc = dev_alloc(h, &L.sg, 2 * I * H / 128)) ||
            (rc = dev_alloc(h, &L.cd, H * I / 2)) || (rc = dev_alloc(h, &L.sd, H * I / 128)))
          return rc;
        L.cu = L.cg + I * H / 2;  // up rows follow the gate rows (codes and scales)
        L.su = L.sg + I * H / 128;
      } else if (q8) {
        if ((rc = dev_alloc(h, &L.qqkv, NQKV * H)) || (rc = dev_alloc(h, &L.sqkv, NQKV * H / 32)) ||
            (rc = dev_alloc(h, &L.qo, H * nq * d)) || (rc = dev_alloc(h, &L.so, H * nq * d / 32)) ||
            (rc = dev_alloc(h, &L.qg, 2 * I * H)) || (rc = dev_alloc(h, &L.sg, 2 * I * H / 32)) ||
            (rc = dev_alloc(h, &L.qd, H * I)) || (rc = dev_alloc(h, &L.sd, H * I / 32)))
          return rc;
        L.qu = L.qg + I * H;  // up rows follow the gate rows (codes and scales)
        L.su = L.sg + I * H / 32;
      } else if ((rc = dev_alloc(h, &L.wqkv, NQKV * H)) || (rc = dev_alloc(h, &L.wo, H * nq * d)) ||
                 (rc = dev_alloc(h, &L.wg, 2 * I * H)) || (rc = dev_alloc(h, &L.wd, H * I))) {
        return rc;
      } else {
        L.wu = L.wg + I * H;  // gate and up rows share one allocation
      }
      if (c.qk_norm && ((rc = dev_alloc(h, &L.q_norm, d)) || (rc = dev_alloc(h, &L.k_norm, d)))) return rc;
      if (c.qkv_bias && (rc = dev_alloc(h, &L.bqkv, NQKV))) return rc;
    }
  }
  HIP_TRY(h, hipMemcpyAsync(h->embed, w->embed, (size_t)c.vocab * H * 2, hipMemcpyDeviceToDevice, s));
  widen(w->final_norm, h->final_norm, H);
  for (int l = 0; l < c.n_layers; ++l) {
    Layer& L = h->layers[l];
    if (q4) {
      // rows [row0, row0 + nrows) of a source matrix [*, K] -> rows from dst_row of the engine's matrix
      auto quant = [&](const void* src, size_t row0, size_t nrows, size_t K, uint8_t* codes, uint16_t* scales,
                       size_t dst_row) {
        launch_quantize_q4(s, (const uint16_t*)src + row0 * K, (int)nrows, (int)K, codes + dst_row * (K / 2),
                           scales + dst_row * (K / 128));
      };
      for (size_t g = 0; g < nkv; ++g) {
        const size_t r = g * (G + 2) * d;
        quant(w->wq[l], g * G * d, G * d, H, L.cqkv, L.sqkv, r);
        quant(w->wk[l], g * d, d, H, L.cqkv, L.sqkv, r + G * d);
        quant(w->wv[l], g * d, d, H, L.cqkv, L.sqkv, r + (G + 1) * d);
      }
      quant(w->wo[l], 0, H, nq * d, L.co, L.so, 0);
      quant(w->w_gate[l], 0, I, H, L.cg, L.sg, 0);
      quant(w->w_up[l], 0, I, H, L.cu, L.su, 0);
      quant(w->w_down[l], 0, H, I, L.cd, L.sd, 0);
    } else if (q8) {
      auto quant = [&](const void* src, size_t row0, size_t nrows, size_t K, int8_t* codes, uint16_t* scales,
                       size_t dst_row) {
        launch_quantize_q8(s, (const uint16_t*)src + row0 * K, (int)nrows, (int)K, codes + dst_row * K,
                           scales + dst_row * (K / 32));
      };
      for (size_t g = 0; g < nkv; ++g) {
        const size_t r = g * (G + 2) * d;
        quant(w->wq[l], g * G * d, G * d, H, L.qqkv, L.sqkv, r);
        quant(w->wk[l], g * d, d, H, L.qqkv, L.sqkv, r + G * d);
        quant(w->wv[l], g * d, d, H, L.qqkv, L.sqkv, r + (G + 1) * d);
      }
      quant(w->wo[l], 0, H, nq * d, L.qo, L.so, 0);
      quant(w->w_gate[l], 0, I, H, L.qg, L.sg, 0);
      quant(w->w_up[l], 0, I, H, L.qu, L.su, 0);
      quant(w->w_down[l], 0, H, I, L.qd, L.sd, 0);
    }
    // fused q|k|v rows, group-major: [kv head g][q heads g*G .. g*G+G-1 | k_g | v_g] x d rows
    for (size_t g = 0; !q4 && !q8 && g < nkv; ++g) {
      uint16_t* dst = L.wqkv + g * (G + 2) * d * H;
      HIP_TRY(h, hipMemcpyAsync(dst, (const uint16_t*)w->wq[l] + g * G * d * H, G * d * H * 2,
                                hipMemcpyDeviceToDevice, s));
      HIP_TRY(h, hipMemcpyAsync(dst + G * d * H, (const uint16_t*)w->wk[l] + g * d * H, d * H * 2,
                                hipMemcpyDeviceToDevice, s));
      HIP_TRY(h, hipMemcpyAsync(dst + (G + 1) * d * H, (const uint16_t*)w->wv[l] + g * d * H, d * H * 2,
                                hipMemcpyDeviceToDevice, s));
    }
    if (!q4 && !q8) {
      HIP_TRY(h, hipMemcpyAsync(L.wo, w->wo[l], H * nq * d * 2, hipMemcpyDeviceToDevice, s));
      HIP_TRY(h, hipMemcpyAsync(L.wg, w->w_gate[l], I * H * 2, hipMemcpyDeviceToDevice, s));
      HIP_TRY(h, hipMemcpyAsync(L.wu, w->w_up[l], I * H * 2, hipMemcpyDeviceToDevice, s));
      HIP_TRY(h, hipMemcpyAsync(L.wd, w->w_down[l], H * I * 2, hipMemcpyDeviceToDevice, s));
    }
    widen(w->attn_norm[l], L.attn_norm, H);
    widen(w->mlp_norm[l], L.mlp_norm, H);
    if (c.qk_norm) {
      widen(w->q_norm[l], L.q_norm, d);
      widen(w->k_norm[l], L.k_norm, d);
    }
    if (c.qkv_bias) {
      for (size_t g = 0; g < nkv; ++g) {
        float* dst = L.bqkv + g * (G + 2) * d;
        widen((const uint16_t*)w->bq[l] + g * G * d, dst, G * d);
        widen((const uint16_t*)w->bk[l] + g * d, dst + G * d, d);
        widen((const uint16_t*)w->bv[l] + g * d, dst + (G + 1) * d, d);
      }
    }
  }
  HIP_TRY(h, hipGetLastError());
  if (h->persistent) {
    std::vector<LayerPtrs> lp(c.n_layers);
    for (int l = 0; l < c.n_layers; ++l) {
      const Layer& L = h->layers[l];
      const bool lo = !h->lora.empty();
      lp[l] = LayerPtrs{L.wqkv, L.bqkv, L.attn_norm, L.mlp_norm, L.q_norm, L.k_norm, L.wo, L.wg, L.wu, L.wd,
                        {L.cqkv, L.co, L.cg, L.cd}, {L.sqkv, L.so, L.sg, L.sd},
                        lo ? h->lora[l].a : nullptr, lo ? h->lora[l].bq : nullptr, lo ? h->lora[l].bv : nullptr};
    }
    PersistConst pc{};
    pc.L = c.n_layers; pc.H = c.hidden; pc.nq = c.n_q_heads; pc.nkv = c.n_kv_heads; pc.I = c.intermediate;
    pc.V = c.vocab; pc.nqkv = (int)NQKV; pc.max_pos = c.max_pos; pc.eps = c.rms_eps; pc.q4 = q4;
    pc.lora_r = h->lora_rank; pc.lora_scale = h->lora_scale;
    pc.embed = h->embed; pc.final_norm = h->final_norm; pc.layers = h->layer_ptrs;
    pc.Kc = h->Kc; pc.Vc = h->Vc; pc.rope_cos = h->rope_cos; pc.rope_sin = h->rope_sin;
    pc.X0 = h->X0; pc.X1 = h->X1; pc.QKV = h->QKVx; pc.PART = h->PART; pc.O = h->Ox; pc.ACT = h->ACT;
    pc.AM = h->AM; pc.TOK = h->TOK; pc.logits = h->logits; pc.xf_out = nullptr; pc.st = h->st; pc.err = h->err_dev;
    pc.trace = h->trace_on ? h->trace : nullptr;
    h->pc_host = pc;
    HIP_TRY(h, hipMemcpyAsync(h->layer_ptrs, lp.data(), lp.size() * sizeof(LayerPtrs), hipMemcpyHostToDevice, s));
    HIP_TRY(h, hipMemcpyAsync(h->pconst, &pc, sizeof(pc), hipMemcpyHostToDevice, s));
  }
  HIP_TRY(h, hipStreamSynchronize(s));
  h->weights = true;
  return qd_reset_kv(h);
}

int qd_reset_kv(qd_handle* h) {
  if (!h) return QD_E_ARG;
  HIP_TRY(h, hipMemsetAsync(h->st, 0, sizeof(DevState), h->stream));
  if (h->err_dev) {  // an abandoned step of the episode that ends here stays counted in err[1]
    hipLaunchKernelGGL(k_fold_err, dim3(1), dim3(64), 0, h->stream, h->err_dev);
    HIP_TRY(h, hipGetLastError());
  }
  if (h->ACT && fill_pairs(h, h->stream) != QD_OK)
    return h->set_err(QD_E_HIP, "hipMemsetAsync of the value-pair buffers failed");
  h->failed = false;
  h->pos = 0;
  h->have_token = false;
  h->cap_rows = 0;
  return QD_OK;
}

int qd_prefill(qd_handle* h, const int32_t* tokens_host, int32_t n, const qd_sampling* sampling, float* logits_dev,
               int32_t* token_dev) {
  if (!h) return QD_E_ARG;
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (!tokens_host) return h->set_err(QD_E_ARG, "tokens is NULL");
  if (n <= 0) return h->set_err(QD_E_ARG, "empty prompt (n <= 0)");
  if (n > h->cfg.max_prefill) return h->set_err(QD_E_RANGE, "n exceeds max_prefill");
  if ((int64_t)h->pos + n > h->cfg.max_pos) return h->set_err(QD_E_RANGE, "position would exceed max_pos");
  for (int i = 0; i < n; ++i)
    if (tokens_host[i] < 0 || tokens_host[i] >= h->cfg.vocab) return h->set_err(QD_E_ARG, "token id out of range");
  int rc = check_sampling(h, sampling);
  if (rc) return rc;
  // the pinned staging buffer may still feed an earlier async copy
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  memcpy(h->tokens_pinned, tokens_host, (size_t)n * sizeof(int32_t));
  HIP_TRY(h, hipMemcpyAsync(h->tokens_dev, h->tokens_pinned, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice,
                            h->stream));
  enqueue_forward(h, n, h->tokens_dev, h->capture_on);
  HIP_TRY(h, hipGetLastError());
  if ((rc = maybe_sample(h, sampling))) return rc;
  h->pos += n;
  h->have_token = true;
  h->cap_rows = h->capture_on ? n : 0;
  return copy_outputs(h, logits_dev, token_dev);
}

int qd_decode_step(qd_handle* h, const qd_sampling* sampling, float* logits_dev, int32_t* token_dev) {
  if (!h) return QD_E_ARG;
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (!h->have_token) return h->set_err(QD_E_STATE, "decode before prefill");
  if (h->pos + 1 > h->cfg.max_pos) return h->set_err(QD_E_RANGE, "position would exceed max_pos");
  int rc = check_sampling(h, sampling);
  if (rc) return rc;
  if (h->failed) return h->set_err(QD_E_STATE, "an earlier decode step was abandoned; call qd_reset_kv");
  if (h->persistent) {
    if (++h->seq >= (1u << 24)) h->seq = 1;
    PersistStep st;
    if (persist_plan(h->pc_host, h->grid, h->pos, h->seq, &st) != 0)
      return h->set_err(QD_E_HIP, "no CU role plan for this decode step");
    const int G = h->cfg.n_q_heads / h->cfg.n_kv_heads;
    if (h->trace_on)  // a traced step writes only the stamps of its CUs' phases
      HIP_TRY(h, hipMemsetAsync(h->trace, 0, (size_t)h->grid * persist_trace_slots(h->cfg.n_layers) * 8, h->stream));
    int e = persist_launch(h->pconst, G, h->hseg, h->cfg.weight_format == QD_W_INT4_G128, h->pc_host.lora_r > 0,
                           h->grid, st, h->stream);
    if (e != 0) return h->set_err(QD_E_HIP, "persistent decode launch failed: " + std::to_string(e));
    if ((rc = maybe_sample(h, sampling))) return rc;
    h->pos += 1;
    h->traced_step = h->trace_on;
    return copy_outputs(h, logits_dev, token_dev);
  }
  if (!h->decode_exec) {
    HIP_TRY(h, hipStreamBeginCapture(h->stream, hipStreamCaptureModeThreadLocal));
    enqueue_forward(h, 1, &h->st->token, false);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(h->stream, &g);
    if (e != hipSuccess) return h->set_err(QD_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    h->decode_graph = g;
    HIP_TRY(h, hipGraphInstantiate(&h->decode_exec, g, nullptr, nullptr, 0));
  }
  HIP_TRY(h, hipGraphLaunch(h->decode_exec, h->stream));
  if ((rc = maybe_sample(h, sampling))) return rc;
  h->pos += 1;
  return copy_outputs(h, logits_dev, token_dev);
}

int qd_verify(qd_handle* h, const int32_t* tokens_host, int32_t m, float* logits_dev, int32_t* choices_dev) {
  if (!h) return QD_E_ARG;
  const qd_config& c = h->cfg;
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (!tokens_host) return h->set_err(QD_E_ARG, "tokens is NULL");
  if (m < 1 || m > QD_VERIFY_MAX) return h->set_err(QD_E_ARG, "m must be in [1, QD_VERIFY_MAX]");
  if (m > c.max_prefill) return h->set_err(QD_E_RANGE, "m exceeds max_prefill");
  if ((int64_t)h->pos + m > c.max_pos) return h->set_err(QD_E_RANGE, "position would exceed max_pos");
  for (int i = 0; i < m; ++i)
    if (tokens_host[i] < 0 || tokens_host[i] >= c.vocab) return h->set_err(QD_E_ARG, "token id out of range");
  if (h->failed) return h->set_err(QD_E_STATE, "an earlier decode step was abandoned; call qd_reset_kv");
  hipStream_t s = h->stream;
  HIP_TRY(h, hipStreamSynchronize(s));  // the pinned staging buffer may still feed an earlier copy
  memcpy(h->tokens_pinned, tokens_host, (size_t)m * sizeof(int32_t));
  HIP_TRY(h, hipMemcpyAsync(h->tokens_dev, h->tokens_pinned, (size_t)m * sizeof(int32_t), hipMemcpyHostToDevice, s));
  // the m rows through the layers (a prefill of m rows), then the final norm
  // and LM head of every row, up to lmhead_rows_per_pass rows per E pass; as
  // one captured graph per (attention mode, m), every position read from the
  // step state
  const int H = c.hidden, V = c.vocab, nblk = lmhead_blocks(V);
  const int mode = m > 1 && m <= kRowAttnMaxRows && h->pos >= kRowAttnMinPos ? 1 : 0;
  hipGraphExec_t& ex = h->verify_exec[mode][m];
  if (!ex) {
    HIP_TRY(h, hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal));
    launch_embed(s, h->embed, h->tokens_dev, m, H, h->x);
    if (m >= kGemmMinRows && c.weight_format != QD_W_Q8_0)
      enqueue_layers_gemm(h, m, false);
    else
      enqueue_layers_gemv(h, m, false);
    int np = nblk;  // partials per row (row stride nblk)
    for (int t0 = 0, tr = lmhead_rows_per_pass(H); t0 < m; t0 += tr) {
      const int tn = std::min(tr, m - t0);
      np = launch_lmhead_rows_bf16(s, h->embed, V, H, h->x + (size_t)t0 * H, tn, h->final_norm, c.rms_eps,
                              h->vlogits + (size_t)t0 * V, h->vpval + (size_t)t0 * nblk, h->vpidx + (size_t)t0 * nblk);
    }
    launch_argmax_rows(s, h->vpval, h->vpidx, nblk, np, m, h->st, h->vchoice);
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(s, &g);
    if (e != hipSuccess) return h->set_err(QD_E_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
    h->verify_graph[mode][m] = g;
    HIP_TRY(h, hipGraphInstantiate(&ex, g, nullptr, nullptr, 0));
  }
  HIP_TRY(h, hipGraphLaunch(ex, s));
  h->pos += m;
  h->have_token = true;
  h->cap_rows = 0;
  if (logits_dev)
    HIP_TRY(h, hipMemcpyAsync(logits_dev, h->vlogits, (size_t)m * V * 4, hipMemcpyDeviceToDevice, s));
  if (choices_dev) HIP_TRY(h, hipMemcpyAsync(choices_dev, h->vchoice, (size_t)m * 4, hipMemcpyDeviceToDevice, s));
  return QD_OK;
}

int qd_rewind(qd_handle* h, int32_t n, int32_t next_token) {
  if (!h) return QD_E_ARG;
  if (n < 0 || n > h->pos) return h->set_err(QD_E_ARG, "n must be in [0, position]");
  if (next_token < 0 || next_token >= h->cfg.vocab) return h->set_err(QD_E_ARG, "token id out of range");
  launch_rewind_state(h->stream, h->st, n, next_token);
  HIP_TRY(h, hipGetLastError());
  h->pos -= n;
  h->have_token = h->pos > 0;
  h->cap_rows = 0;
  return QD_OK;
}

int qd_decode_steps(qd_handle* h, int32_t n, const qd_sampling* sampling, float* logits_dev, int32_t* tokens_dev) {
  if (!h) return QD_E_ARG;
  if (n < 1) return h->set_err(QD_E_ARG, "n must be >= 1");
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (!h->have_token) return h->set_err(QD_E_STATE, "decode before prefill");
  if ((int64_t)h->pos + n > h->cfg.max_pos) return h->set_err(QD_E_RANGE, "position would exceed max_pos");
  int rc = check_sampling(h, sampling);
  if (rc) return rc;
  if (h->failed) return h->set_err(QD_E_STATE, "an earlier decode step was abandoned; call qd_reset_kv");
  const bool greedy = !sampling || sampling->temperature <= 0.f || sampling->top_k == 1;
  if (!h->persistent || !greedy || h->trace_on) {  // one step per launch, all enqueued without a host wait
    for (int i = 0; i < n; ++i) {
      if ((rc = qd_decode_step(h, sampling, i + 1 == n ? logits_dev : nullptr, tokens_dev ? tokens_dev + i : nullptr)))
        return rc;
    }
    return QD_OK;
  }
  // greedy persistent: runs of steps with one split count per launch
  const int G = h->cfg.n_q_heads / h->cfg.n_kv_heads;
  for (int done = 0; done < n;) {
    const int m = persist_batch_len(h->pc_host, h->grid, h->pos, std::min(n - done, kMaxStepsPerLaunch));
    if (h->seq + m >= (1u << 24)) h->seq = 0;  // tags of the launch's steps: seq + 1 .. seq + m
    PersistStep st;
    if (persist_plan(h->pc_host, h->grid, h->pos, h->seq + 1, &st) != 0)
      return h->set_err(QD_E_HIP, "no CU role plan for this decode step");
    st.nsteps = m;
    st.tokens_out = tokens_dev ? tokens_dev + done : nullptr;
    int e = persist_launch(h->pconst, G, h->hseg, h->cfg.weight_format == QD_W_INT4_G128, h->pc_host.lora_r > 0,
                           h->grid, st, h->stream);
    if (e != 0) return h->set_err(QD_E_HIP, "persistent decode launch failed: " + std::to_string(e));
    h->seq += m;
    h->pos += m;
    done += m;
  }
  h->traced_step = false;
  return copy_outputs(h, logits_dev, nullptr);
}

// The persistent step's copy of the adapter's rank and scale (its plan gives
// the LoRA-down CU only while one is installed); ordered on the stream before
// the next step.
static int sync_persist_lora(qd_handle* h) {
  if (!h->persistent || !h->weights) return QD_OK;
  h->pc_host.lora_r = h->lora_rank;
  h->pc_host.lora_scale = h->lora_scale;
  HIP_TRY(h, hipMemcpyAsync(h->pconst, &h->pc_host, sizeof(PersistConst), hipMemcpyHostToDevice, h->stream));
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  return QD_OK;
}

int qd_set_lora(qd_handle* h, const qd_lora* lora) {
  if (!h) return QD_E_ARG;
  if (!lora) return h->set_err(QD_E_ARG, "lora is NULL");
  if (lora->struct_size != sizeof(qd_lora)) return h->set_err(QD_E_ABI, "qd_lora.struct_size mismatch");
  const qd_config& c = h->cfg;
  if (c.lora_rank_max == 0) return h->set_err(QD_E_STATE, "LoRA not enabled (lora_rank_max = 0)");
  if (lora->rank < 1 || lora->rank > c.lora_rank_max) return h->set_err(QD_E_ARG, "rank must be in [1, lora_rank_max]");
  if (!std::isfinite(lora->alpha)) return h->set_err(QD_E_ARG, "alpha must be finite");
  if (!lora->a_q || !lora->b_q || !lora->a_v || !lora->b_v) return h->set_err(QD_E_ARG, "a LoRA array is NULL");
  for (int l = 0; l < c.n_layers; ++l)
    if (!lora->a_q[l] || !lora->b_q[l] || !lora->a_v[l] || !lora->b_v[l])
      return h->set_err(QD_E_ARG, "NULL LoRA pointer in layer " + std::to_string(l));
  const size_t r = lora->rank, H = c.hidden, d = c.head_dim;
  hipStream_t s = h->stream;
  for (int l = 0; l < c.n_layers; ++l) {
    const LoraLayer& A = h->lora[l];
    HIP_TRY(h, hipMemcpyAsync(A.a, lora->a_q[l], r * H * 2, hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, hipMemcpyAsync(A.a + r * H, lora->a_v[l], r * H * 2, hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, hipMemcpyAsync(A.bq, lora->b_q[l], (size_t)c.n_q_heads * d * r * 2, hipMemcpyDeviceToDevice, s));
    HIP_TRY(h, hipMemcpyAsync(A.bv, lora->b_v[l], (size_t)c.n_kv_heads * d * r * 2, hipMemcpyDeviceToDevice, s));
  }
  HIP_TRY(h, hipStreamSynchronize(s));
  h->lora_rank = (int)r;
  h->lora_scale = lora->alpha / (float)r;
  drop_decode_graph(h);  // the next decode step captures the adapter's kernels
  return sync_persist_lora(h);
}

int qd_clear_lora(qd_handle* h) {
  if (!h) return QD_E_ARG;
  if (h->lora_rank) {
    HIP_TRY(h, hipStreamSynchronize(h->stream));  // the captured step may still be running
    h->lora_rank = 0;
    drop_decode_graph(h);
    return sync_persist_lora(h);
  }
  return QD_OK;
}

int qd_enable_capture(qd_handle* h, int32_t enable) {
  if (!h) return QD_E_ARG;
  if (enable && !h->cap) {
    const qd_config& c = h->cfg;
    size_t n = (size_t)(c.n_layers + 1) * c.max_prefill * c.hidden + c.hidden + c.vocab;
    int rc = dev_alloc(h, &h->cap, n);
    if (rc) return rc;
  }
  h->capture_on = enable != 0;
  return QD_OK;
}

int qd_get_capture(qd_handle* h, int32_t what, int32_t layer, float* out_host, size_t capacity_elems,
                   size_t* written_elems) {
  if (!h) return QD_E_ARG;
  if (!out_host) return h->set_err(QD_E_ARG, "out_host is NULL");
  if (h->cap_rows == 0 || !h->cap) return h->set_err(QD_E_STATE, "nothing captured");
  const qd_config& c = h->cfg;
  const size_t H = c.hidden, rows = h->cap_rows;
  const float* src = nullptr;
  size_t n = 0;
  switch (what) {
    case QD_CAP_EMBED: src = h->cap; n = rows * H; break;
    case QD_CAP_LAYER_OUT:
      if (layer < 0 || layer >= c.n_layers) return h->set_err(QD_E_ARG, "layer out of range");
      src = h->cap + (size_t)(layer + 1) * c.max_prefill * H;
      n = rows * H;
      break;
    case QD_CAP_FINAL_NORM: src = h->cap + (size_t)(c.n_layers + 1) * c.max_prefill * H; n = H; break;
    case QD_CAP_LOGITS: src = h->cap + (size_t)(c.n_layers + 1) * c.max_prefill * H + H; n = c.vocab; break;
    default: return h->set_err(QD_E_ARG, "unknown capture point");
  }
  if (capacity_elems < n) return h->set_err(QD_E_ARG, "capacity smaller than the capture");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  HIP_TRY(h, hipMemcpy(out_host, src, n * 4, hipMemcpyDeviceToHost));
  if (written_elems) *written_elems = n;
  return QD_OK;
}

int qd_enable_phase_trace(qd_handle* h, int32_t enable) {
  if (!h) return QD_E_ARG;
  if (!h->persistent) return h->set_err(QD_E_STATE, "phase trace needs the persistent decode step");
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (enable && !h->trace) {
    const size_t n = (size_t)h->grid * persist_trace_slots(h->cfg.n_layers);
    int rc = dev_alloc(h, &h->trace, n);
    if (rc) return rc;
    HIP_TRY(h, hipMemset(h->trace, 0, n * 8));
  }
  h->trace_on = enable != 0;
  h->pc_host.trace = h->trace_on ? h->trace : nullptr;
  HIP_TRY(h, hipMemcpyAsync(h->pconst, &h->pc_host, sizeof(PersistConst), hipMemcpyHostToDevice, h->stream));
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  h->traced_step = false;
  return QD_OK;
}

int qd_get_phase_trace(qd_handle* h, uint64_t* out_host, size_t capacity_elems, size_t* written_elems,
                       int32_t* n_cu) {
  if (!h) return QD_E_ARG;
  if (!out_host) return h->set_err(QD_E_ARG, "out_host is NULL");
  if (!h->persistent || !h->trace || !h->traced_step) return h->set_err(QD_E_STATE, "no traced decode step");
  const size_t n = (size_t)h->grid * persist_trace_slots(h->cfg.n_layers);
  if (capacity_elems < n) return h->set_err(QD_E_ARG, "capacity smaller than the trace");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  HIP_TRY(h, hipMemcpy(out_host, h->trace, n * 8, hipMemcpyDeviceToHost));
  if (written_elems) *written_elems = n;
  if (n_cu) *n_cu = h->grid;
  return QD_OK;
}

int qd_get_exchange(qd_handle* h, int32_t which, float* out_host, size_t capacity_elems, size_t* written_elems) {
  if (!h) return QD_E_ARG;
  if (!out_host) return h->set_err(QD_E_ARG, "out_host is NULL");
  if (!h->persistent) return h->set_err(QD_E_STATE, "exchange buffers belong to the persistent decode step");
  const qd_config& c = h->cfg;
  const uint64_t* src = nullptr;
  size_t n = 0;
  bool pairs = false;
  switch (which) {
    case QD_XCH_X0: src = h->X0; n = c.hidden; break;
    case QD_XCH_X1: src = h->X1; n = c.hidden; break;
    case QD_XCH_QKV: src = h->QKVx; n = (size_t)qkv_rows(c); break;
    case QD_XCH_ATTN: src = h->Ox; n = (size_t)c.n_q_heads * c.head_dim; pairs = true; break;
    case QD_XCH_ACT: src = h->ACT; n = c.intermediate; pairs = true; break;
    default: return h->set_err(QD_E_ARG, "unknown exchange buffer");
  }
  if (capacity_elems < n) return h->set_err(QD_E_ARG, "capacity smaller than the buffer");
  std::vector<uint64_t> words(pairs ? n / 2 : n);
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  HIP_TRY(h, hipMemcpy(words.data(), src, words.size() * 8, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < words.size(); ++i) {
    if (pairs) {  // {tag16 | a24 | b24}: the top 24 bits of two floats
      const uint32_t a = (uint32_t)((words[i] >> 24) & 0xFFFFFFu) << 8, b = (uint32_t)(words[i] & 0xFFFFFFu) << 8;
      memcpy(out_host + 2 * i, &a, 4);
      memcpy(out_host + 2 * i + 1, &b, 4);
    } else {
      const uint32_t a = (uint32_t)words[i];
      memcpy(out_host + i, &a, 4);
    }
  }
  if (written_elems) *written_elems = n;
  return QD_OK;
}

int qd_get_quantized(qd_handle* h, int32_t layer, int32_t which, int8_t* codes_host, size_t codes_capacity,
                     uint16_t* scales_host, size_t scales_capacity) {
  if (!h) return QD_E_ARG;
  const qd_config& c = h->cfg;
  const bool q4 = c.weight_format == QD_W_INT4_G128;
  if (!q4 && c.weight_format != QD_W_Q8_0) return h->set_err(QD_E_STATE, "the handle does not hold quantised weights");
  if (!h->weights) return h->set_err(QD_E_STATE, "weights not loaded");
  if (!codes_host || !scales_host) return h->set_err(QD_E_ARG, "output pointer is NULL");
  if (layer < 0 || layer >= c.n_layers) return h->set_err(QD_E_ARG, "layer out of range");
  const size_t H = c.hidden, d = c.head_dim, I = c.intermediate, nq = c.n_q_heads, nkv = c.n_kv_heads;
  const size_t G = nq / nkv, gs = q4 ? 128 : 32;  // columns per scale
  const Layer& L = h->layers[layer];
  // (source matrix, its rows, K) and, for q/k/v, where each kv group's rows sit in the fused matrix
  const uint8_t* cs = nullptr;
  const uint16_t* ss = nullptr;
  size_t N = 0, K = 0, src_rows = 0, per_group = 0, group_off = 0;
  auto codes_of = [&](const uint8_t* c4, const int8_t* c8) { return q4 ? c4 : reinterpret_cast<const uint8_t*>(c8); };
  switch (which) {
    case QD_PROJ_Q: cs = codes_of(L.cqkv, L.qqkv); ss = L.sqkv; N = nq * d; K = H; per_group = G * d; group_off = 0; break;
    case QD_PROJ_K: cs = codes_of(L.cqkv, L.qqkv); ss = L.sqkv; N = nkv * d; K = H; per_group = d; group_off = G * d; break;
    case QD_PROJ_V: cs = codes_of(L.cqkv, L.qqkv); ss = L.sqkv; N = nkv * d; K = H; per_group = d; group_off = (G + 1) * d; break;
    case QD_PROJ_O: cs = codes_of(L.co, L.qo); ss = L.so; N = H; K = nq * d; break;
    case QD_PROJ_GATE: cs = codes_of(L.cg, L.qg); ss = L.sg; N = I; K = H; break;
    case QD_PROJ_UP: cs = codes_of(L.cu, L.qu); ss = L.su; N = I; K = H; break;
    case QD_PROJ_DOWN: cs = codes_of(L.cd, L.qd); ss = L.sd; N = H; K = I; break;
    default: return h->set_err(QD_E_ARG, "unknown projection");
  }
  if (codes_capacity < N * K || scales_capacity < N * (K / gs))
    return h->set_err(QD_E_ARG, "capacity smaller than the matrix");
  src_rows = per_group ? (size_t)qkv_rows(c) : N;
  const size_t row_bytes = q4 ? K / 2 : K;
  std::vector<uint8_t> codes(src_rows * row_bytes);
  std::vector<uint16_t> scales(src_rows * K / gs);
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  HIP_TRY(h, hipMemcpy(codes.data(), cs, codes.size(), hipMemcpyDeviceToHost));
  HIP_TRY(h, hipMemcpy(scales.data(), ss, scales.size() * 2, hipMemcpyDeviceToHost));
  for (size_t n = 0; n < N; ++n) {
    const size_t r = per_group ? (n / per_group) * (G + 2) * d + group_off + n % per_group : n;
    for (size_t k = 0; k < K; ++k) {
      if (q4) {
        const uint8_t b = codes[r * row_bytes + k / 2];
        codes_host[n * K + k] = (int8_t)((k & 1 ? b >> 4 : b & 15) - 8);
      } else {
        codes_host[n * K + k] = (int8_t)codes[r * row_bytes + k];
      }
    }
    for (size_t g = 0; g < K / gs; ++g) scales_host[n * (K / gs) + g] = scales[r * (K / gs) + g];
  }
  return QD_OK;
}

int qd_sync_token(qd_handle* h, int32_t* token_host) {
  if (!h) return QD_E_ARG;
  if (!token_host) return h->set_err(QD_E_ARG, "token_host is NULL");
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  if (h->persistent) {
    uint32_t e = 0;
    HIP_TRY(h, hipMemcpy(&e, h->err_dev, 4, hipMemcpyDeviceToHost));
    if (e) {
      h->failed = true;
      return h->set_err(QD_E_HIP, "a decode step was abandoned (device-side wait timed out)");
    }
  }
  DevState st;
  HIP_TRY(h, hipMemcpy(&st, h->st, sizeof(st), hipMemcpyDeviceToHost));
  *token_host = st.token;
  return QD_OK;
}

int qd_get_abandoned(qd_handle* h, int64_t* count_out) {
  if (!h) return QD_E_ARG;
  if (!count_out) return h->set_err(QD_E_ARG, "count_out is NULL");
  *count_out = 0;
  HIP_TRY(h, hipStreamSynchronize(h->stream));
  if (h->err_dev) {
    uint32_t e[2] = {0, 0};
    HIP_TRY(h, hipMemcpy(e, h->err_dev, 8, hipMemcpyDeviceToHost));
    *count_out = (int64_t)e[1] + (e[0] != 0 ? 1 : 0);
  }
  return QD_OK;
}

int qd_get_position(const qd_handle* h, int32_t* pos_out) {
  if (!h || !pos_out) return QD_E_ARG;
  *pos_out = h->pos;
  return QD_OK;
}

void qd_destroy(qd_handle* h) {
  if (!h) return;
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  free_all(h);
  delete h;
}

}  // extern "C"
