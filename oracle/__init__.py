"""CPU oracle for the single-sequence forward step of a Qwen3-style decoder.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
HIP library never calls it, and it shares no code with the HIP library: the
only common module is ``synth`` (seeded input draws, no model arithmetic).

The oracle is the plain definition of the model, written in numpy float64:
weights are the bf16 values (or the int4 group-128 / Q8_0 codes times their
fp16 scales) widened exactly to float64, and every activation, reduction and the
attention cache are float64.  Library matmuls are used as single steps; there
is no blocking, fusion or reordering beyond the definition.

Sources followed (cited by page title and section in each function):
  * "Failed Star / fs — Forward pass → logits" (M2): gather, RMSNorm,
    QK-norm, RoPE, GQA causal attention, o_proj and SwiGLU residual blocks,
    final norm, last row, tied embedding head; [out,in] weight rows.
  * "flashmoon demo/README.md — Qwen3-0.6B inference": f32 KV cache, greedy
    (temp = 0) and temperature/top-k/top-p sampling.
  * "EMBERGLASS (qwen-webgpu-lora) README": int4 group-128 weights, rank-r
    LoRA on the projections, batched prefill equal to sequential decode, and
    the optional reduced-precision (bf16) KV cache.
  * "SuperKittens pull request #7", the Q8_0 commit: int8 weights in blocks
    of 32 with an fp16 scale.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, hand-worked examples (``tests/golden/``), invariants and special cases.
"""
from .model import OracleModel, rmsnorm, rope_rotate, causal_gqa_attention, silu, swiglu_mlp, argmax_lowest  # noqa: F401
from .model import round_bf16  # noqa: F401
from .quant import quantize_int4_g128, dequantize_int4_g128, quantize_q8_0, dequantize_q8_0  # noqa: F401
from .sampling import splitmix64_output, uniform_for_step, sample_top_k_top_p  # noqa: F401
