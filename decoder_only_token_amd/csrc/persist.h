// Persistent single-kernel decode step (internal to libqd).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

// Per-layer weight pointers, stored in device memory for the persistent kernel.
struct LayerPtrs {
  const uint16_t* wqkv;  // [(nq + 2 nkv) d][H] bf16
  const float* bqkv;     // [(nq + 2 nkv) d] or null
  const float* attn_norm;
  const float* mlp_norm;
  const float* q_norm;  // [d] or null (no QK-norm)
  const float* k_norm;
  const uint16_t* wo;  // [H][nq d]
  const uint16_t* wg;  // [I][H]
  const uint16_t* wu;  // [I][H]
  const uint16_t* wd;  // [H][I]
  // int4 group-128 weights of the four projections q|k|v, o, gate (+ up), down,
  // in that order (codes u8 [rows][in / 2], fp16 scales [rows][in / 128], same
  // row order as the bf16 matrices above, which are then null); the up rows'
  // codes and scales follow the gate rows' in one allocation each
  const uint8_t* qcode[4];
  const uint16_t* qscale[4];
  // LoRA factors (bf16, rank r = PersistConst::lora_r): down rows [A_q; A_v]
  // [2 r][H], up rows B_q [nq d][r] and B_v [nkv d][r] (original head order)
  const uint16_t* lora_a;
  const uint16_t* lora_bq;
  const uint16_t* lora_bv;
};

// Everything the decode kernel needs that does not change from step to step.
// The exchange buffers hold 64-bit words {f32 value | tag << 32}.
struct PersistConst {
  int L, H, nq, nkv, I, V, nqkv, max_pos;
  int q4;  // 1: the projections are int4 group-128 (LayerPtrs c* / s*)
  int lora_r;        // 0: no adapter; else its rank (one more CU in the QKV role)
  float lora_scale;  // alpha / r
  float eps;
  const uint16_t* embed;
  const float* final_norm;
  const LayerPtrs* layers;
  float* Kc;  // [L][nkv][max_pos][128]
  float* Vc;
  const float* rope_cos;  // [max_pos][64]
  const float* rope_sin;
  uint64_t* X0;    // [H] residual entering a layer
  uint64_t* X1;    // [H] residual after attention
  uint64_t* QKV;   // [nqkv + 2 lora_r]: q|k|v rows, then the LoRA down products u_q, u_v
  uint64_t* PART;  // [nq][S][130] split partials {m, l, o[128]}
  uint64_t* O;     // [nq * 64] attention output, value pairs
  uint64_t* ACT;   // [I / 2] SwiGLU activations, value pairs
  uint64_t* AM;    // [grid][2] per-CU {best logit, best id (bit pattern)}
  uint64_t* TOK;   // [1] the token a step chose, for the launch's next step
  float* logits;   // [V]
  float* xf_out;   // [H] final-normed row (optional)
  DevState* st;
  uint32_t* err;   // err[0] != 0: a wait timed out; the step was abandoned
  uint64_t* trace; // optional [grid][(5 L + 2) * 8] real-time stamps of the last step
};

// Trace stamps per phase (100 MHz real-time counter), per CU, by thread 0:
//   0 starts polling the phase input       1 the input is in LDS (after the barrier)
//   2 finished its dot products            3 outputs published
//   5 next slice requested (phase done)    7 kernel start (phase 0 only); 4, 6 unused
constexpr int kTraceSlots = 8;
__host__ __device__ inline int persist_trace_slots(int L) { return (5 * L + 2) * kTraceSlots; }

// One decode step's launch plan: the attention splits and the CU ranges of
// the five roles (role r runs on blocks [start[r], start[r + 1]): QKV rows
// (with an adapter, the role's last CU computes the LoRA down products),
// attention items (kv head, head group, split), o_proj rows, gate/up row
// pairs, down rows).
struct PersistStep {
  int pos;       // position of the new token
  uint32_t seq;  // step number in the tags (1 .. 2^24 - 1)
  int S, chunk;  // splits per kv head, positions per split
  int X;         // head groups per kv head: attention items = nkv X S
  int start[6];
  // decode steps in this launch (positions pos .. pos + nsteps - 1, tags seq
  // .. seq + nsteps - 1), all with this plan's CU roles and split count S
  // (each step's splits one position longer, as its own plan would cut them);
  // tokens_out (device, optional) receives the nsteps tokens
  int nsteps;
  int32_t* tokens_out;
};

size_t persist_smem_bytes();
int persist_prepare(int G, int hseg, int q4, int lora);  // lora: the instantiation with an adapter
// Plans the step at position pos for `grid` CUs; 0 on success, -1 if the
// grid cannot hold the five roles.
int persist_plan(const PersistConst& pc, int grid, int pos, uint32_t seq, PersistStep* out);
// The number of steps from position pos (at most nmax) whose plans have the
// same split count S, so one launch can run them with one plan.
int persist_batch_len(const PersistConst& pc, int grid, int pos, int nmax);
int persist_launch(const PersistConst* dev_const, int G, int hseg, int q4, int lora, int grid, const PersistStep& st,
                   hipStream_t s);
