"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module only *draws* inputs: model shapes, random bf16 weights, random
prompt token IDs, LoRA factors and sampling settings.  It holds none of the
forward-pass arithmetic; the oracle (``oracle/``) and the HIP library each
implement that on their own.

Workloads (model shape + prompt/decode lengths) follow the five synthetic
workloads this project is measured on.  No public dataset is used: weights
are N(0, 0.02) draws rounded to bf16, prompts are uniform random token IDs.
The pages this library follows ran real Qwen checkpoints on real prompts,
which are not available here; the seeded draws stand in for them with the
same shapes.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

SEED_WEIGHTS = 0
SEED_PROMPT = 1
SEED_SAMPLING = 2
SEED_LORA = 3

W_BF16 = 0
W_INT4_G128 = 1
W_Q8_0 = 2  # int8 blocks of 32 with an fp16 scale


@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    rope_theta: float = 1e6
    rms_eps: float = 1e-6
    qk_norm: bool = True
    qkv_bias: bool = False
    weight_format: int = W_BF16
    max_pos: int = 2048


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    prompt_len: int
    decode_steps: int          # number of decode_step calls after the prefill token
    max_prefill: int
    lora_rank: int = 0
    lora_alpha: float = 0.0
    temperature: float = 0.0   # 0 = greedy
    top_k: int = 0
    top_p: float = 1.0


TINY = ModelShape("tiny-qwen3", 2, 1024, 16, 8, 128, 3072, 4096, max_pos=64)
QWEN3_06B = ModelShape("qwen3-0.6b", 28, 1024, 16, 8, 128, 3072, 151936, max_pos=2048)
QWEN25_3B_INT4 = ModelShape("qwen2.5-3b-int4g128", 36, 2048, 16, 2, 128, 11008, 151936,
                            qk_norm=False, qkv_bias=True, weight_format=W_INT4_G128, max_pos=4096)
QWEN25_3B_INT4_16K = dataclasses.replace(QWEN25_3B_INT4, name="qwen2.5-3b-int4g128-16k", max_pos=16384)
# Small int4 models of the 3B family's structure (8 query heads per kv head,
# q/k/v bias, no QK-norm).  Their projection widths end partway into a
# 2048-column pass (1024, 1408) or run one pass and a ragged rest (2432).
TINY_INT4 = ModelShape("tiny-int4g128", 2, 1024, 16, 2, 128, 1408, 4096, qk_norm=False, qkv_bias=True,
                       weight_format=W_INT4_G128, max_pos=256)
TINY_INT4_WIDE = ModelShape("tiny-int4g128-wide", 2, 2048, 16, 2, 128, 2432, 4096, qk_norm=False, qkv_bias=True,
                            weight_format=W_INT4_G128, max_pos=256)

# Q8_0 models: the 0.6B shape and a tiny one whose widths end partway into a
# 1024-column pass (1408) or run one pass and a ragged rest (2432)
QWEN3_06B_Q8 = dataclasses.replace(QWEN3_06B, name="qwen3-0.6b-q8_0", weight_format=W_Q8_0)
TINY_Q8 = ModelShape("tiny-q8_0", 2, 1024, 16, 8, 128, 1408, 4096, weight_format=W_Q8_0, max_pos=256)
TINY_Q8_WIDE = ModelShape("tiny-q8_0-wide", 2, 2048, 16, 2, 128, 2432, 4096, qk_norm=False, qkv_bias=True,
                          weight_format=W_Q8_0, max_pos=256)

WORKLOADS: Dict[str, Workload] = {
    # 8-token prompt, 16 greedy decode steps
    "tiny": Workload("tiny", TINY, 8, 16, 64),
    # 5-token prompt, 128 greedy decode steps, MAXPOS 2048
    "qwen3-0.6b": Workload("qwen3-0.6b", QWEN3_06B, 5, 128, 512),
    # 512-token batched prefill, decode until the KV cache holds 2048 positions;
    # greedy, and T=0.7 / top-k 40 / top-p 0.9 sampling
    "qwen3-0.6b-long": Workload("qwen3-0.6b-long", QWEN3_06B, 512, 2048 - 512, 512,
                                temperature=0.7, top_k=40, top_p=0.9),
    # 256-token prompt, decode to context 4096
    "qwen2.5-3b-int4": Workload("qwen2.5-3b-int4", QWEN25_3B_INT4, 256, 4096 - 256, 512),
    # the 0.6B model with Q8_0 projection weights: 5-token prompt, 128 greedy steps
    "qwen3-0.6b-q8_0": Workload("qwen3-0.6b-q8_0", QWEN3_06B_Q8, 5, 128, 512),
    # 8192-token prefill with rank-16 LoRA on q/v, decode to context 16384
    "qwen2.5-3b-int4-lora": Workload("qwen2.5-3b-int4-lora", QWEN25_3B_INT4_16K, 8192, 16384 - 8192, 8192,
                                     lora_rank=16, lora_alpha=32.0),
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even (input preparation only)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)  # wraps only for NaN bit patterns, fixed below
    r >>= 16
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep NaN a (quiet) NaN
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return bf16_round(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def layer_tensor_names(shape: ModelShape) -> List[str]:
    names = ["attn_norm", "wq", "wk", "wv"]
    if shape.qkv_bias:
        names += ["bq", "bk", "bv"]
    if shape.qk_norm:
        names += ["q_norm", "k_norm"]
    names += ["wo", "mlp_norm", "w_gate", "w_up", "w_down"]
    return names


def tensor_shape(shape: ModelShape, name: str):
    H, d, I = shape.hidden, shape.head_dim, shape.intermediate
    q, kv = shape.n_q_heads * d, shape.n_kv_heads * d
    return {
        "attn_norm": (H,), "mlp_norm": (H,), "q_norm": (d,), "k_norm": (d,),
        "wq": (q, H), "wk": (kv, H), "wv": (kv, H), "bq": (q,), "bk": (kv,), "bv": (kv,),
        "wo": (H, q), "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I),
    }[name]


def make_weights(shape: ModelShape, seed: int = SEED_WEIGHTS, std: float = 0.02,
                 random_gains: bool = False) -> Dict[str, object]:
    """Draw a full weight set as bf16 bit patterns.

    Order of draws (fixed): embed [V,H]; then per layer, in order, every matrix
    and bias of ``layer_tensor_names``; norm gains are 1.0 and not drawn unless
    ``random_gains`` is set (then each gain vector is 1 + N(0, 0.1), drawn in
    its place in the same order, and the final gain after the last layer).
    Returns {"embed": u16[V,H], "final_norm": u16[H], "layers": [ {name: u16[...]}, ... ]}.
    """
    rng = np.random.default_rng(seed)
    H = shape.hidden
    out: Dict[str, object] = {"embed": _normal_bf16(rng, (shape.vocab, H), std)}
    layers = []
    ones = lambda n: bf16_round(np.ones(n, np.float32))  # noqa: E731
    for _ in range(shape.n_layers):
        lw = {}
        for name in layer_tensor_names(shape):
            shp = tensor_shape(shape, name)
            if name.endswith("_norm"):
                if random_gains:
                    lw[name] = bf16_round(1.0 + 0.1 * rng.standard_normal(shp, dtype=np.float32))
                else:
                    lw[name] = ones(shp)
            else:
                lw[name] = _normal_bf16(rng, shp, std)
        layers.append(lw)
    out["layers"] = layers
    if random_gains:
        out["final_norm"] = bf16_round(1.0 + 0.1 * rng.standard_normal((H,), dtype=np.float32))
    else:
        out["final_norm"] = ones((H,))
    return out


def make_lora(shape: ModelShape, rank: int, seed: int = SEED_LORA, std: float = 0.01) -> List[Dict[str, np.ndarray]]:
    """Rank-r LoRA factors on q_proj and v_proj for every layer, bf16 bit patterns.

    Per layer, drawn in order: a_q [r,H], b_q [nq*d, r], a_v [r,H], b_v [nkv*d, r].
    """
    rng = np.random.default_rng(seed)
    H, d = shape.hidden, shape.head_dim
    res = []
    for _ in range(shape.n_layers):
        res.append({
            "a_q": _normal_bf16(rng, (rank, H), std),
            "b_q": _normal_bf16(rng, (shape.n_q_heads * d, rank), std),
            "a_v": _normal_bf16(rng, (rank, H), std),
            "b_v": _normal_bf16(rng, (shape.n_kv_heads * d, rank), std),
        })
    return res


def make_prompt(vocab: int, n: int, seed: int = SEED_PROMPT) -> np.ndarray:
    """n uniform random token IDs in [0, vocab), int32."""
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int32)


def make_logits(vocab: int, seed: int, scale: float = 3.0, step: Optional[float] = None) -> np.ndarray:
    """f32 logits ~ N(0, scale^2); with `step`, rounded to multiples of it so
    that many entries tie (for the lowest-id tie rule)."""
    x = np.random.default_rng(seed).standard_normal(vocab) * scale
    if step:
        x = np.round(x / step) * step
    return x.astype(np.float32)


def scaled_shape(shape: ModelShape, **kw) -> ModelShape:
    return dataclasses.replace(shape, **kw)


def weight_bytes(shape: ModelShape, lora_rank: int = 0) -> Dict[str, int]:
    """Algorithmic bytes one decode step reads from the weights, by kind.

    bf16 matrices: 2 bytes per element.  int4 group-128: half a byte per code plus
    a 2-byte fp16 scale per 128 codes.  Q8_0: one byte per code plus a 2-byte
    fp16 scale per 32 codes.  Norm gains and biases are bf16.  The tied
    embedding table is bf16 and read once for the LM head (plus one row gathered).
    """
    H, d, I, L = shape.hidden, shape.head_dim, shape.intermediate, shape.n_layers
    nq, nkv, V = shape.n_q_heads, shape.n_kv_heads, shape.vocab
    lin = (nq * d + 2 * nkv * d) * H + H * nq * d + 2 * I * H + H * I
    if shape.weight_format == W_BF16:
        mat = 2 * lin
    elif shape.weight_format == W_Q8_0:
        mat = lin + 2 * (lin // 32)
    else:
        mat = lin // 2 + 2 * (lin // 128)
    small = 2 * (2 * H) + (2 * 2 * d if shape.qk_norm else 0) + (2 * (nq * d + 2 * nkv * d) if shape.qkv_bias else 0)
    lora = 0
    if lora_rank:
        lora = 2 * lora_rank * (2 * H + nq * d + nkv * d)
    return {
        "layers": L * (mat + small),
        "lora": L * lora,
        "lm_head": 2 * V * H + 2 * H,
        "embed_row": 2 * H,
    }


def kv_bytes_per_position(shape: ModelShape) -> int:
    """f32 K and V for one position across all layers."""
    return shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * 4


def make_weights_device(shape: ModelShape, seed: int = SEED_WEIGHTS, std: float = 0.02, device: str = "cuda"):
    """The same weight set structure drawn on the GPU (torch's counter-based
    Philox generator seeded with `seed`, N(0, std) in float32 rounded to bf16
    by torch's round-to-nearest-even conversion), returned as int16 device
    tensors holding the bf16 bit patterns; gains 1.0.  Same draw order as
    make_weights.  Used where only the shapes matter (benchmark inputs); the
    parity tests use make_weights, whose draws the oracle also sees."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(*shp):
        t = torch.randn(*shp, generator=g, device=device, dtype=torch.float32) * std
        return t.to(torch.bfloat16).view(torch.int16)

    ones = lambda n: torch.ones(n, device=device, dtype=torch.bfloat16).view(torch.int16)  # noqa: E731
    out = {"embed": normal(shape.vocab, shape.hidden)}
    layers = []
    for _ in range(shape.n_layers):
        lw = {}
        for name in layer_tensor_names(shape):
            shp = tensor_shape(shape, name)
            lw[name] = ones(shp[0]) if name.endswith("_norm") else normal(*shp)
        layers.append(lw)
    out["layers"] = layers
    out["final_norm"] = ones(shape.hidden)
    return out


def make_lora_device(shape: ModelShape, rank: int, seed: int = SEED_LORA, std: float = 0.01, device: str = "cuda"):
    """LoRA factors as in make_lora, drawn on the GPU (see make_weights_device)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    H, d = shape.hidden, shape.head_dim

    def normal(*shp):
        t = torch.randn(*shp, generator=g, device=device, dtype=torch.float32) * std
        return t.to(torch.bfloat16).view(torch.int16)

    return [{"a_q": normal(rank, H), "b_q": normal(shape.n_q_heads * d, rank), "a_v": normal(rank, H),
             "b_v": normal(shape.n_kv_heads * d, rank)} for _ in range(shape.n_layers)]


def device_to_host(weights_dev, layers=None):
    """bf16 bit patterns (numpy uint16) of a device weight set, all layers or the given ones."""
    import numpy as np
    h = lambda t: t.cpu().numpy().view(np.uint16)  # noqa: E731
    idx = range(len(weights_dev["layers"])) if layers is None else layers
    return {"embed": h(weights_dev["embed"]), "final_norm": h(weights_dev["final_norm"]),
            "layers": [{k: h(v) for k, v in weights_dev["layers"][i].items()} for i in idx]}
