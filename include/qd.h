/*
 * qd.h — C ABI of the MI355X (gfx950) single-sequence decoder-step library.
 *
 * The library computes the forward step of a Qwen3-style decoder-only
 * transformer for one sequence: embedding gather, then per layer RMSNorm,
 * Q/K/V projection (+bias, +LoRA), per-head QK-RMSNorm, RoPE applied as K is
 * written to an f32 KV cache, causal grouped-query attention, o_proj and
 * residual, RMSNorm, SwiGLU gate/up/down and residual; then the final norm,
 * the tied-embedding LM head and an on-GPU argmax or top-k/top-p draw.
 *
 * Sources (page title, section):
 *   - "Failed Star / fs — Forward pass → logits": the block order, [out,in]
 *     weight rows, the tied head borrowing the embedding table, the last-row
 *     projection, rejection of empty or over-long prompts before any work.
 *   - "flashmoon demo/README.md — Qwen3-0.6B inference": f32 KV cache, RoPE
 *     fused into the cache write, in-place SiLU and residual, argmax on the GPU
 *     so only the token crosses to the host; temperature 0 means greedy;
 *     MAXPOS sizing of the cache.
 *   - "EMBERGLASS (qwen-webgpu-lora) README": int4 group-128 weights quantised
 *     on the way to the GPU, split-K decode attention, live LoRA that restores
 *     the base bit-for-bit when cleared, maxCtx / maxPrefillT options.
 *   - "SuperKittens PR #7 (qwen3: 0.6B correctness + 2.6x decode speedup)":
 *     a C ABI of config and weight structs behind a ctypes binding (and the
 *     struct-size mismatches that motivate struct_size / abi_version here),
 *     the capture call that must fail for what was not captured and must not
 *     overrun the caller's buffer, seq-major vs head-major layout at T >= 2.
 *
 * Conventions
 *   - Every call returns an int status: QD_OK (0) or a negative QD_E_* code.
 *     qd_last_error() returns a text reason for the last failure on a handle
 *     (qd_last_error(NULL): of the last failed handle-free call).
 *   - Arguments are checked before any state change or GPU work; a failed
 *     call leaves the handle as it was.
 *   - "device pointer" = memory allocated on the handle's GPU (hipMalloc or
 *     a torch CUDA tensor).  "host pointer" = ordinary process memory.
 *   - GPU work is enqueued on the hipStream_t given to qd_create and is
 *     asynchronous unless stated; qd_sync_token() synchronises.
 *   - Not thread-safe: one handle must not be used by two threads at once.
 */
#ifndef QD_H
#define QD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QD_ABI_VERSION 2

typedef struct qd_handle qd_handle; /* opaque; owns every device buffer it allocates */

enum {
  QD_OK = 0,
  QD_E_ARG = -1,   /* bad argument: NULL pointer, bad shape, n <= 0, capacity too small */
  QD_E_ABI = -2,   /* struct_size or abi_version does not match this library */
  QD_E_STATE = -3, /* call not valid now (no weights, decode before prefill, nothing captured) */
  QD_E_RANGE = -4, /* position would exceed max_pos, or n exceeds max_prefill */
  QD_E_OOM = -5,   /* device allocation failed */
  QD_E_HIP = -6    /* a HIP runtime call failed */
};

enum { QD_W_BF16 = 0, QD_W_INT4_G128 = 1, QD_W_Q8_0 = 2 };

/* Model and engine shape.  Copied by qd_create. */
typedef struct {
  uint32_t struct_size; /* = sizeof(qd_config) */
  uint32_t abi_version; /* = QD_ABI_VERSION */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, vocab;
  float rope_theta; /* RoPE base; pair j of a head turns by pos * theta^(-2j/head_dim) */
  float rms_eps;    /* epsilon inside the RMSNorm square root */
  uint8_t qk_norm;        /* 1: per-head RMSNorm of q and k before RoPE */
  uint8_t qkv_bias;       /* 1: q/k/v projections carry a bias */
  uint8_t tie_embeddings; /* must be 1: the LM head is the embedding table */
  uint8_t weight_format;  /* QD_W_BF16, QD_W_INT4_G128 or QD_W_Q8_0 (projections only; E stays bf16).
                             QD_W_Q8_0 ("SuperKittens pull request #7", the Q8_0 commit: int8 in
                             blocks of 32 columns with an fp16 scale, quantised at qd_load_weights)
                             needs decode_path QD_DECODE_GRAPH; its prefills run the GEMV kernels
                             on tiles of up to 8 rows */
  int32_t max_pos;        /* KV-cache capacity in positions */
  int32_t max_prefill;    /* largest n accepted by one qd_prefill call */
  int32_t lora_rank_max;  /* 0 disables LoRA; else the largest rank qd_set_lora accepts (<= 64;
                             QD_DECODE_PERSISTENT: ceil(r / 4) * ceil(hidden / 512) <= 24) */
  int32_t decode_path;    /* QD_DECODE_PERSISTENT (one kernel per decode step, one workgroup per CU,
                             at most 254 layers,
                             all resident at once: the device must not be running other work
                             meanwhile, else a step can be abandoned after its bounded wait)
                             or QD_DECODE_GRAPH (one kernel per operation, replayed as a hipGraph) */
  int32_t kv_format;      /* QD_KV_F32 (keys and values as computed) or QD_KV_BF16 ("EMBERGLASS
                             (qwen-webgpu-lora) README", Context window & prefill sizes: a quantised
                             KV cache would roughly halve its size): every key (after RoPE) and value
                             is rounded to bf16 (nearest, ties to even) when it is stored, and
                             attention reads it back from the cache, the new rows included.  Half
                             the cache bytes; QD_DECODE_GRAPH only. */
} qd_config;

enum { QD_DECODE_PERSISTENT = 0, QD_DECODE_GRAPH = 1 };
enum { QD_KV_F32 = 0, QD_KV_BF16 = 1 };

/* Weights: device pointers to bf16 (uint16 bit patterns), row-major [out, in].
 * Per-layer fields are HOST arrays of n_layers device pointers.  Shapes:
 *   embed [vocab, hidden], final_norm [hidden], attn_norm/mlp_norm [hidden],
 *   q_norm/k_norm [head_dim] (read only when qk_norm), wq [nq*d, hidden],
 *   wk/wv [nkv*d, hidden], bq [nq*d], bk/bv [nkv*d] (read only when qkv_bias),
 *   wo [hidden, nq*d], w_gate/w_up [intermediate, hidden], w_down [hidden, intermediate].
 * Everything is copied (or, for QD_W_INT4_G128, quantised) into buffers the
 * handle owns; the caller's memory is only borrowed during the call. */
typedef struct {
  uint32_t struct_size; /* = sizeof(qd_weights) */
  const void* embed;
  const void* final_norm;
  const void* lm_head; /* must be NULL (tied) */
  const void* const* attn_norm;
  const void* const* mlp_norm;
  const void* const* q_norm;
  const void* const* k_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* bq;
  const void* const* bk;
  const void* const* bv;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
} qd_weights;

/* Token choice.  temperature <= 0 (or a NULL qd_sampling*) means greedy argmax
 * with ties to the lowest id.  Otherwise: keep the top_k logits (by value, then
 * lowest id; top_k <= 0 or > 64 is rejected), softmax at `temperature`, keep
 * the shortest prefix whose mass before each kept entry is < top_p, and pick
 * with the uniform u = (SplitMix64 output number (step+1) from state `seed`) >> 40
 * divided by 2^24, where step counts tokens chosen since the last qd_reset_kv
 * (0 = the token chosen by the first qd_prefill). */
typedef struct {
  uint32_t struct_size; /* = sizeof(qd_sampling) */
  float temperature;
  int32_t top_k;
  float top_p;
  uint64_t seed;
} qd_sampling;

/* Rank-r LoRA on q_proj and v_proj: q += (alpha/r) B_q (A_q h), v += (alpha/r) B_v (A_v h),
 * h = the attention-normed input.  HOST arrays of n_layers device pointers to bf16:
 * a_q/a_v [r, hidden], b_q [nq*d, r], b_v [nkv*d, r].  Copied into the handle. */
typedef struct {
  uint32_t struct_size; /* = sizeof(qd_lora) */
  int32_t rank;
  float alpha;
  const void* const* a_q;
  const void* const* b_q;
  const void* const* a_v;
  const void* const* b_v;
} qd_lora;

/* Capture points for layer-by-layer comparison (what argument of qd_get_capture). */
enum {
  QD_CAP_EMBED = 0,      /* f32 [n, hidden]: gathered rows of the last prefill */
  QD_CAP_LAYER_OUT = 1,  /* f32 [n, hidden]: residual after layer `layer` */
  QD_CAP_FINAL_NORM = 2, /* f32 [hidden]: final-normed last row */
  QD_CAP_LOGITS = 3      /* f32 [vocab]: logits of the last row */
};

/* Validate *cfg (before any HIP call), then allocate the KV cache
 * ([n_layers][n_kv_heads][max_pos][head_dim] f32 for K and for V), workspaces
 * and RoPE tables on the current HIP device (see below).  The persistent decode
 * step runs one workgroup per compute unit; the environment variable
 * QD_PERSIST_CUS = n (read here) limits it to n workgroups (diagnostics and
 * tests: more rows per CU, slices larger than the registers loaded ahead).
 *
 * Validate *cfg (before any HIP call), then allocate the KV cache
 * ([n_layers][n_kv_heads][max_pos][head_dim] f32 for K and for V), workspaces
 * and RoPE tables on the current HIP device.  hip_stream is a hipStream_t
 * that all later work is enqueued on; NULL makes the handle create (and own)
 * a non-blocking stream of its own, which the legacy default stream does not
 * wait for: then read outputs after qd_sync_token() or a device-wide
 * synchronisation.  (A decode step is captured as a graph, which the legacy
 * default stream cannot hold.)
 * On success *out receives a new handle.  Errors: QD_E_ARG, QD_E_ABI, QD_E_OOM, QD_E_HIP. */
int qd_create(const qd_config* cfg, void* hip_stream, qd_handle** out);

/* Copy (or quantise) every weight into the handle; synchronous with respect to
 * the caller's pointers (they may be freed on return).  Resets the KV cache.
 * Errors: QD_E_ARG (NULL field, lm_head not NULL), QD_E_ABI, QD_E_HIP. */
int qd_load_weights(qd_handle* h, const qd_weights* w);

/* Empty the KV cache: position := 0, step := 0.  The LoRA state is kept. */
int qd_reset_kv(qd_handle* h);

/* Append n prompt tokens (host int32 array, ids in [0, vocab)) at the current
 * position in one batched pass, then choose the next token from the last
 * row's logits.  Requires 1 <= n <= max_prefill and position + n <= max_pos.
 * logits_dev (device f32 [vocab]) and token_dev (device int32 [1]) are
 * optional outputs, written asynchronously.  The chosen token stays on the
 * device as the input of the next qd_decode_step.
 * Errors: QD_E_ARG (NULL tokens, n <= 0, id out of range), QD_E_RANGE, QD_E_STATE (no weights). */
int qd_prefill(qd_handle* h, const int32_t* tokens_host, int32_t n, const qd_sampling* sampling,
               float* logits_dev, int32_t* token_dev);

/* One decode step: consume the device-resident last token at the current
 * position, write its K/V, and choose the next token.  Needs a prior
 * qd_prefill since the last reset and position + 1 <= max_pos.
 * Errors: QD_E_STATE, QD_E_RANGE, QD_E_ARG (bad sampling). */
int qd_decode_step(qd_handle* h, const qd_sampling* sampling, float* logits_dev, int32_t* token_dev);

/* n decode steps in one call, the token each step chooses feeding the next on
 * the device, with no host wait in between ("EMBERGLASS (qwen-webgpu-lora)
 * README", why it is fast: a GPU-resident batched decode loop, argmax to
 * embedding on the GPU, one sync per batch).  tokens_dev (device int32[n],
 * optional) receives the n tokens in order; logits_dev (optional) the last
 * step's logits.  Greedy on QD_DECODE_PERSISTENT: one kernel launch runs the
 * steps whose plans share one attention split count (a launch runs up to 64
 * steps; a longer or split-count-crossing run takes a few launches); each
 * step's results are bit for bit those of qd_decode_step.  Sampling,
 * QD_DECODE_GRAPH or an enabled phase trace: one launch per step.
 * Errors: as qd_decode_step; QD_E_ARG (n < 1), QD_E_RANGE (pos + n > max_pos). */
int qd_decode_steps(qd_handle* h, int32_t n, const qd_sampling* sampling, float* logits_dev, int32_t* tokens_dev);

/* Speculative verification ("flashmoon demo/README.md", Known limitations:
 * no speculative decode, a single sequence; here for that one sequence).
 * Consumes the m host tokens tokens_host[0 .. m) at positions pos .. pos + m - 1,
 * as a prefill of m rows, and makes the greedy choice after every row:
 * choices_dev[i] (device int32[m], optional) = argmax of the logits after
 * tokens[0 .. i] (lowest id on ties), the choice a greedy decode step would
 * make there; logits_dev (device f32[m][vocab], optional) receives the rows'
 * logits.  The projections run as for a prefill of m rows (GEMV kernels that
 * read each weight once for up to 8 rows; matrix cores from 16 rows) and the
 * LM head reads the embedding table once for up to 8 rows.  Afterwards the
 * position is pos + m and the next input token is choices[m - 1], as after m
 * decode steps.  With tokens = [the next input token, d1, .., d(m-1)] (drafts)
 * and a = the number of leading drafts equal to the choice before them
 * (d(i) == choices[i - 1]), the a + 1 tokens d1 .. da, choices[a] are exactly
 * those of a + 1 greedy decode steps; qd_rewind(h, m - 1 - a, choices[a])
 * then drops the rejected rows.
 * Errors: QD_E_STATE (no weights), QD_E_ARG (NULL tokens, m outside
 * [1, QD_VERIFY_MAX], token out of range), QD_E_RANGE (m > max_prefill or
 * pos + m > max_pos). */
#define QD_VERIFY_MAX 16
int qd_verify(qd_handle* h, const int32_t* tokens_host, int32_t m, float* logits_dev, int32_t* choices_dev);

/* Drop the last n positions of the cache (position -= n; their K/V rows are
 * overwritten by later steps) and make next_token the next input token.
 * Stream-ordered, no synchronisation.
 * Errors: QD_E_ARG (n outside [0, position], token out of range). */
int qd_rewind(qd_handle* h, int32_t n, int32_t next_token);

/* Install (copy) a LoRA adapter ("EMBERGLASS (qwen-webgpu-lora) README", LoRA
 * sections: a live low-rank adapter on q_proj and v_proj).  Needs
 * lora_rank_max >= 1 at qd_create; rank must be in 1..lora_rank_max and alpha
 * finite.  On the persistent decode step one more CU computes the down
 * products A h and the attention items add the up products.  The adapter applies to every
 * later prefill and decode step; the KV cache is kept.  Synchronises the
 * stream.  qd_clear_lora removes it: the adapter's kernels no longer run, so
 * outputs are bit-for-bit those of the base model.
 * Errors: QD_E_STATE (lora_rank_max = 0), QD_E_ARG (rank, alpha, NULL array
 * or layer pointer), QD_E_ABI, QD_E_HIP. */
int qd_set_lora(qd_handle* h, const qd_lora* lora);
int qd_clear_lora(qd_handle* h);

/* Copy a capture point of the most recent qd_prefill into out_host (host
 * f32, capacity_elems elements).  Captures are recorded only while enabled
 * with qd_enable_capture(h, 1).  Errors: QD_E_STATE if that point was not
 * captured, QD_E_ARG if capacity_elems is smaller than the capture. */
int qd_enable_capture(qd_handle* h, int32_t enable);
int qd_get_capture(qd_handle* h, int32_t what, int32_t layer, float* out_host, size_t capacity_elems,
                   size_t* written_elems);

/* Phase trace of the persistent decode step (diagnostics).  While enabled,
 * every CU records 100 MHz real-time counter stamps, 8 slots per phase p
 * (per layer l: 5l = QKV, 5l+1 = attention, 5l+2 = o_proj, 5l+3 = gate/up,
 * 5l+4 = down; then 5L = LM head, 5L+1 = final argmax on CU 0): slot 8p+0 =
 * starts waiting for the phase input, 8p+1 = input ready, 8p+3 = dot products
 * done, 8p+5 = phase outputs written; slot 7 = kernel start; other slots are
 * left zero.  qd_get_phase_trace copies the stamps of the last decode step,
 * laid out [cu][8 (5L+2)], into out_host (uint64, capacity_elems elements)
 * and reports the CU count.
 * Errors: QD_E_STATE when the handle does not use the persistent decode step
 * or no traced step has run; QD_E_ARG when capacity_elems is too small. */
int qd_enable_phase_trace(qd_handle* h, int32_t enable);
int qd_get_phase_trace(qd_handle* h, uint64_t* out_host, size_t capacity_elems, size_t* written_elems,
                       int32_t* n_cu);

/* Exchange buffers of the persistent decode step (diagnostics): after a step
 * they hold the LAST layer's values of that step (which argument):
 *   QD_XCH_X0   f32 [hidden]        residual after the last layer (the final norm's input)
 *   QD_XCH_X1   f32 [hidden]        residual after the last layer's attention block
 *   QD_XCH_QKV  f32 [(nq+2nkv) d]   raw q|k|v projection (+bias; an adapter's up products are
 *                                   added later, by the attention items), kv-group-major
 *                                   ([kv head g][q heads of g | k_g | v_g] x d)
 *   QD_XCH_ATTN f32 [nq d]          attention output, 16 significant bits
 *   QD_XCH_ACT  f32 [intermediate]  SiLU(gate) * up, 16 significant bits
 * qd_get_exchange synchronises the stream and copies one of them into
 * out_host.  Errors: QD_E_STATE (not the persistent path), QD_E_ARG (NULL
 * output, unknown buffer, capacity too small), QD_E_HIP. */
enum { QD_XCH_X0 = 0, QD_XCH_X1 = 1, QD_XCH_QKV = 2, QD_XCH_ATTN = 3, QD_XCH_ACT = 4 };
int qd_get_exchange(qd_handle* h, int32_t which, float* out_host, size_t capacity_elems, size_t* written_elems);

/* Projections of a layer, for qd_get_quantized. */
enum { QD_PROJ_Q = 0, QD_PROJ_K = 1, QD_PROJ_V = 2, QD_PROJ_O = 3, QD_PROJ_GATE = 4, QD_PROJ_UP = 5, QD_PROJ_DOWN = 6 };

/* Read back the encoding that qd_load_weights made of one projection of layer
 * `layer`, in the caller's [out, in] order whatever the library's own layout.
 * QD_W_INT4_G128 ("EMBERGLASS (qwen-webgpu-lora) README", "Note on weights":
 * int4 in groups of 128, quantised on the way to the GPU): B = 128, codes in
 * [-7, 7]; QD_W_Q8_0 ("SuperKittens pull request #7", the Q8_0 commit): B =
 * 32, codes in [-127, 127].
 *   codes_host  int8 [N][K]                              (codes_capacity >= N K)
 *   scales_host fp16 bit patterns [N][K / B]             (scales_capacity >= N K / B)
 * with N x K the shape of that projection (qd_weights); the weight of row n,
 * column k is codes[n][k] * scale[n][k / B].  Synchronises the stream.
 * Errors: QD_E_STATE (weights not loaded, or bf16 weights), QD_E_ARG (NULL
 * output, bad layer or projection, capacity too small), QD_E_HIP. */
int qd_get_quantized(qd_handle* h, int32_t layer, int32_t which, int8_t* codes_host, size_t codes_capacity,
                     uint16_t* scales_host, size_t scales_capacity);

/* Synchronise the stream and read the device-resident last token.
 * Errors: QD_E_HIP when a persistent decode step since the last qd_reset_kv was
 * abandoned (its bounded device-side wait timed out: the device was shared);
 * later decode steps then fail with QD_E_STATE until qd_reset_kv. */
int qd_sync_token(qd_handle* h, int32_t* token_host);

/* Synchronise the stream and report in *count_out the number of cache
 * episodes (spans between qd_reset_kv calls, the current one included) in
 * which a persistent decode step was abandoned since qd_create.  qd_reset_kv
 * does not clear this count, so a caller can check a whole run of episodes
 * once, outside its timed work.  Always 0 for QD_DECODE_GRAPH.
 * Errors: QD_E_ARG (NULL count_out), QD_E_HIP. */
int qd_get_abandoned(qd_handle* h, int64_t* count_out);

/* Current position (number of tokens in the KV cache), host-side mirror. */
int qd_get_position(const qd_handle* h, int32_t* pos_out);

/* Token choice over logits the caller already holds, without a handle: the
 * same greedy / top-k / temperature / top-p rule as qd_sampling above
 * ("flashmoon demo/README.md — Qwen3-0.6B inference", Quick start: greedy at
 * temperature 0, else temperature, top-k and top-p; "EMBERGLASS
 * (qwen-webgpu-lora)" decoding notes: the choice stays on the GPU).
 *   logits_dev     device pointer, `vocab` f32 logits.
 *   vocab          1 .. 524288 entries; top_k must not exceed it, and the
 *                  merge's lists must fit its LDS: (ceil(vocab / 1024) + 1)
 *                  * top_k <= 20480 (top_k <= 39 at the largest vocab).
 *   sampling       NULL or temperature <= 0: greedy (ties to the lowest id);
 *                  else top_k in [1, 64], top_p in (0, 1].
 *   step           draw counter: u comes from SplitMix64 output number
 *                  (step + 1) from state sampling->seed (ignored when greedy).
 *   token_dev      device pointer, receives the chosen id (int32).
 *   workspace_dev  device scratch of at least qd_sample_workspace_bytes()
 *                  bytes, 4-byte aligned, owned by the caller; it holds the
 *                  per-slice top-k lists and needs no initial contents.
 *   hip_stream     the hipStream_t to enqueue on (NULL: the null stream), on
 *                  the device current at the call.
 * Asynchronous: two kernels on hip_stream; allocates nothing.  Calls that
 * share a workspace must be ordered on one stream.
 * Errors (nothing enqueued): QD_E_ARG (NULL pointer, bad vocab / top_k /
 * top_p / temperature, workspace too small or misaligned), QD_E_ABI
 * (sampling->struct_size), QD_E_HIP; the reason is qd_last_error(NULL) on the
 * calling thread. */
size_t qd_sample_workspace_bytes(int32_t vocab, const qd_sampling* sampling); /* 0: invalid arguments */
int qd_sample_logits(const float* logits_dev, int32_t vocab, const qd_sampling* sampling, uint64_t step,
                     int32_t* token_dev, void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* qd_sample_logits without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Its scratch is a file-scope device array
 * of 160 KiB per GPU (enough for every supported vocab and top_k), which the
 * library keeps until the process ends; the first call on a device looks up
 * its address.  Calls on one GPU share that array, and it keeps the last
 * call's contents (no call needs it cleared): calls that overlap on one GPU
 * (different streams, or different threads without ordering) race.
 * Arguments, results and errors as qd_sample_logits; allocates nothing. */
int qd_sample_logits_static(const float* logits_dev, int32_t vocab, const qd_sampling* sampling, uint64_t step,
                            int32_t* token_dev, void* hip_stream);

/* Reason of the handle's last failure; with h == NULL, of the last failed
 * handle-free call (qd_sample_*) on the calling thread. */
const char* qd_last_error(const qd_handle* h);
void qd_destroy(qd_handle* h);

size_t qd_sizeof_config(void);
size_t qd_sizeof_weights(void);
size_t qd_sizeof_sampling(void);
size_t qd_sizeof_lora(void);

#ifdef __cplusplus
}
#endif
#endif /* QD_H */
