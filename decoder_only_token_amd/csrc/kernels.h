// Host-side launchers of the gfx950 decoder-step kernels (internal to libqd).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Device-resident step state: the decode graph reads pos/token from here, so
// one captured graph serves every position.
struct DevState {
  int32_t pos;    // tokens already in the KV cache
  int32_t token;  // last chosen token (input of the next decode step)
  int32_t step;   // tokens chosen since the last reset (sampling counter)
  int32_t pad;
};

#define GEMV_MAX_T 8   // input rows handled per GEMV launch
#define GEMV_RPW 4     // output rows per wave (plain GEMV)
#define GATEUP_RPW 2   // output rows per wave (gate/up pair)
#define LMHEAD_RPW 4   // vocabulary rows per wave (LM head)
#define LMHEAD_ROWS 8  // input rows of one multi-row LM head pass

void launch_embed(hipStream_t s, const uint16_t* E, const int32_t* tok, int T, int H, float* x);
// (ncu = compute units of the GPU, used to size the grid)
void launch_gemv_bf16(hipStream_t s, const uint16_t* W, int N, int K, const float* x, int ldx, int T,
                      const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate, int ncu);
void launch_gemv_gateup_bf16(hipStream_t s, const uint16_t* Wg, const uint16_t* Wu, int N, int K, const float* x,
                             int ldx, int T, const float* gain, float eps, float* a, int lda, int ncu);
int lmhead_blocks(int V);
// Final norm + tied LM head of one row with per-workgroup argmax partials;
// returns the number of partials written (<= lmhead_blocks(V)).
int launch_lmhead_bf16(hipStream_t s, const uint16_t* E, int V, int H, const float* x, const float* gain, float eps,
                       float* logits, float* part_val, int32_t* part_idx, float* xf_out);
// Speculative verification: final norm + LM head for T <= lmhead_rows_per_pass(H)
// rows with per-row logits [T][V] and argmax partials at row stride
// lmhead_blocks(V) (the count per row is returned);
// the per-row choices (advancing the step state by T); dropping positions.
int lmhead_rows_per_pass(int H);
int launch_lmhead_rows_bf16(hipStream_t s, const uint16_t* E, int V, int H, const float* x, int T, const float* gain,
                             float eps, float* logits, float* part_val, int32_t* part_idx);
void launch_argmax_rows(hipStream_t s, const float* part_val, const int32_t* part_idx, int nblk, int nparts, int T,
                        DevState* st, int32_t* choice);
void launch_rewind_state(hipStream_t s, DevState* st, int n, int32_t token);
void launch_argmax_final(hipStream_t s, const float* part_val, const int32_t* part_idx, int nparts, DevState* st,
                         int advance, int32_t* token_out);
// The adapter's up products of a batch of rows: u [T][ldu] (u_q then u_v),
// B_q [nq d][r], B_v [nkv d][r] bf16; u == nullptr: no adapter.
struct LoraRows {
  const float* u = nullptr;
  int ldu = 0;
  const uint16_t* bq = nullptr;
  const uint16_t* bv = nullptr;
  int r = 0;
  float scale = 0.f;
};
// The adapter's down products of a batch (T <= 16 rows, K a multiple of 1024):
// u[t][o] = A[o] . (gain * x_t / rms(x_t)), A bf16 [n][K]; false when not covered.
bool launch_lora_down_rows(hipStream_t s, const uint16_t* A, int n, int K, const float* x, int ldx, int T,
                           const float* gain, float eps, float* u, int ldu);
void launch_qk_rope_kv(hipStream_t s, const float* qkv, int ldqkv, int T, int nq, int nkv, int d, const float* qn,
                       const float* kn, float eps, const float* cos_t, const float* sin_t, const DevState* st,
                       float* q_out, void* Kc, void* Vc, int max_pos, int kv_bf16, const LoraRows& lr);
// Decode attention for one new row (attn.hip), from the raw q|k|v projection
// row (group-major): QK-norm (gains may be null), RoPE, the cache write of the
// new k / v, then S splits of length max(cmin, ceil(ctx / S)); part holds
// nq * S * (d + 2) floats.  The row sits at position st->pos + row (row > 0:
// the rows of a short batch, one launch each, in order).
int attn_decode_splits(int max_pos, int nkv, int ncu, int cmin);
void launch_attention_decode(hipStream_t s, const float* qkv, const float* qn, const float* kn, float eps,
                             const float* cos_t, const float* sin_t, int nq, int nkv, void* Kc, void* Vc,
                             int kv_bf16, int max_pos, const DevState* st, int S, int cmin, float* part, float* o_out,
                             const float* lora_u = nullptr, const uint16_t* lora_bq = nullptr,
                             const uint16_t* lora_bv = nullptr, int lora_r = 0, float lora_scale = 0.f, int row = 0);

// Causal attention of T >= 2 new rows (attn.hip), rows at positions pos .. pos + T - 1.
// Split form for short batches at long contexts: the positions cut into S
// splits as the decode attention cuts them, partials part[T][nq][S][D + 2],
// merged into o_out[T][nq D]; q and the new rows' K/V already in place.
void launch_attention_rows_split(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc, const void* Vc,
                                 int kv_bf16, int max_pos, const DevState* st, int S, int cmin, float* part,
                                 float* o_out);
// With `part`, batches whose query tiles do not fill the CUs run the split
// form over attn_prefill_splits(T, ...) splits (partials part[T][nq][S][D + 2])
// and a merge.  oh / ol (optional): the output's bf16 halves too, at the same
// indices (the o_proj input split).
int attn_prefill_splits(int T, int nq, int nkv, int ncu);
void launch_attention_prefill(hipStream_t s, const float* q, int T, int nq, int nkv, const void* Kc, const void* Vc,
                              int kv_bf16, int max_pos, const DevState* st, float* o_out, int ldo, int ncu,
                              float* part = nullptr, int cmin = 16, uint16_t* oh = nullptr, uint16_t* ol = nullptr);

// Top-k / temperature / top-p sampling over the logits (sample.hip); the token
// goes to the device step state, which the greedy pass has already advanced.
int sample_lists(int V);
bool sample_supported(int V, int K);
int sample_prepare();  // with the device current
void launch_sample(hipStream_t s, const float* logits, int V, int K, float temperature, float top_p, uint64_t seed,
                   float* part_val, int32_t* part_idx, DevState* st, uint64_t step, int32_t* token_out);
const char* sample_free_error();

// Batched prefill projections on the matrix cores (gemm.hip).  X rows are
// split into bf16 hi/lo halves (after RMSNorm with gains when `gain` is set),
// then C[T, N] = (Xh + Xl) W[N, K]^T with one of three epilogues.
enum { GEMM_STORE = 0, GEMM_ADD = 1, GEMM_GATEUP = 2 };
bool gemm_supported(int K);
void launch_split_rows(hipStream_t s, const float* x, int ldx, int T, int K, const float* gain, float eps,
                       uint16_t* xh, uint16_t* xl);
// ws: split-K workspace of ws_floats floats (gemm_workspace_floats of the
// largest product); ncu = compute units of the GPU.
size_t gemm_workspace_floats(int T, int K, int N, int ncu);
// ch / cl (gate | up only, optional): the bf16 halves of the output too, as
// k_split_rows would make them from it.
void launch_gemm_hilo(hipStream_t s, int epi, const uint16_t* xh, const uint16_t* xl, int T, int K, const uint16_t* W,
                      const uint16_t* W2, int N, const float* bias, float* C, int ldc, float* ws, size_t ws_floats,
                      int ncu, uint16_t* ch = nullptr, uint16_t* cl = nullptr);
// W given as int4 group-128 codes [N][K / 2] and fp16 scales [N][K / 128]
// (q4.hip layout); K a multiple of 128.  W2 / SW2: the up matrix of GEMM_GATEUP.
void launch_gemm_q4(hipStream_t s, int epi, const uint16_t* xh, const uint16_t* xl, int T, int K, const uint8_t* W,
                    const uint16_t* SW, const uint8_t* W2, const uint16_t* SW2, int N, const float* bias, float* C,
                    int ldc, float* ws, size_t ws_floats, int ncu, uint16_t* ch = nullptr, uint16_t* cl = nullptr);

// int4 group-128 weights (q4.hip): quantiser run at weight load, and the
// GEMVs of decode and short prefills (same contracts as the bf16 GEMVs;
// ncu = compute units, used to size the grid).
void launch_quantize_q4(hipStream_t s, const uint16_t* src, int nrows, int K, uint8_t* codes, uint16_t* scales);
int q4_gemv_t_tile(int K);
// Single-row (decode) int4 GEMVs on the int8 matrix cores, the input split into
// three 7-bit pieces (error <= 2^-20 of the row's largest input); false when
// the shape is not covered (K not a multiple of 128 or above 12288; gate/up:
// K above 2048).
bool q4m_gemv(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x,
              const float* gain, float eps, const float* bias, float* y, int accumulate);
bool q4m_gateup(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su, int N,
                int K, const float* x, const float* gain, float eps, float* a);
// The same for 2 to q4mr_rows(K) rows at once (row strides ldx, ldy / lda); the
// codes are read once for every row; false when the shape or T is not covered.
// q4mr_rows: rows per launch for K columns (8 or 4), or 0 when not covered.
int q4mr_rows(int K, bool gateup);
bool q4mr_gemv(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
               int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate);
bool q4mr_gateup(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su, int N,
                 int K, const float* x, int ldx, int T, const float* gain, float eps, float* a, int lda);
void launch_gemv_q4(hipStream_t s, const uint8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
                    int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate,
                    int ncu,
                    const uint16_t* xw = nullptr, int xn = 0, float* xy = nullptr, int ldxy = 0);
void launch_gemv_gateup_q4(hipStream_t s, const uint8_t* cg, const uint16_t* sg, const uint8_t* cu, const uint16_t* su,
                           int N, int K, const float* x, int ldx, int T, const float* gain, float eps, float* a,
                           int lda, int ncu);

// Q8_0 weights (q8.hip): int8 codes [N][K] and fp16 scales [N][K / 32]; the
// quantiser run at weight load and the GEMVs of decode and short prefills
// (same contracts as the int4 GEMVs).
void launch_quantize_q8(hipStream_t s, const uint16_t* src, int nrows, int K, int8_t* codes, uint16_t* scales);
int q8_gemv_t_tile(int K);
void launch_gemv_q8(hipStream_t s, const int8_t* codes, const uint16_t* scales, int N, int K, const float* x, int ldx,
                    int T, const float* gain, float eps, const float* bias, float* y, int ldy, int accumulate,
                    int ncu);
void launch_gemv_gateup_q8(hipStream_t s, const int8_t* cg, const uint16_t* sg, const int8_t* cu, const uint16_t* su,
                           int N, int K, const float* x, int ldx, int T, const float* gain, float eps, float* a,
                           int lda, int ncu);

