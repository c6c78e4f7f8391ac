"""Oracle model: the plain float64 definition of a Qwen3-style decoder forward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is called
by the HIP library, and nothing here calls it.

Layout conventions (from "Failed Star / fs — Forward pass → logits", section
"One matrix, no hidden machinery"): every linear weight is stored [out, in]
and applied as ``y = x @ W.T``; the embedding is a row gather; the output
projection borrows the tied embedding table as a [V, H] linear.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

from .quant import quantize_int4_g128, dequantize_int4_g128, quantize_q8_0, dequantize_q8_0

_PROJ = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
_W_INT4_G128 = 1
_W_Q8_0 = 2


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns -> float64, exact (bf16 is the top half of an IEEE float32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def widen_bf16_f32(bits) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (8 significant bits), ties to even, as
    float64.  A reduced-precision KV cache ("EMBERGLASS (qwen-webgpu-lora)
    README", Context window & prefill sizes: the f32 KV could be quantised)
    stores every key and value this way.  Written with frexp/ldexp: x = m 2^e
    with m in [0.5, 1), and m is rounded to a multiple of 2^-8."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm over the last axis: g_j * x_j / sqrt(mean_k x_k^2 + eps).

    "Failed Star / fs — Forward pass → logits", figure of the block and the
    FINAL NORM step: each sublayer reads a row-normalised copy of the bus.  The
    epsilon sits inside the square root (plain reading; the page gives no formula).
    """
    ms = np.mean(np.square(x), axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def rope_angles(positions: np.ndarray, d: int, theta: float) -> np.ndarray:
    """phi[i, j] = position_i * theta^(-2j/d) for the d/2 rotation pairs, in float64."""
    j = np.arange(d // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_rotate(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding with half-split pairs (x_j, x_{j+d/2}).

    x has shape [n, heads, d] and row i sits at absolute position positions[i].
    Each pair is rotated by phi = position * theta^(-2j/d):
    (a, b) -> (a cos phi - b sin phi, b cos phi + a sin phi).
    "Failed Star / fs — Forward pass → logits", block figure ("QK-norm · RoPE");
    the pairing convention is the Qwen one (reading: half-split, not interleaved).
    """
    d = x.shape[-1]
    half = d // 2
    ang = rope_angles(positions, d, theta)
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Causal grouped-query attention.

    q [n, nq, d] holds queries at absolute positions q_pos; k, v [T, nkv, d]
    hold keys/values for positions 0..T-1.  Query head h uses kv head
    g = h // (nq / nkv) (consecutive query heads share a kv head).  Scores are
    q.k / sqrt(d); a query at position p sees keys 0..p inclusive; softmax with
    the row maximum subtracted; output is the probability-weighted sum of v.
    "Failed Star / fs — Forward pass → logits", block figure ("GQA causal attention").
    """
    n, nq, d = q.shape
    T, nkv, _ = k.shape
    group = nq // nkv
    out = np.empty((n, nq, d), dtype=np.float64)
    future = np.arange(T)[None, :] > np.asarray(q_pos)[:, None]
    scale = 1.0 / math.sqrt(d)
    for h in range(nq):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T) * scale
        s = np.where(future, -np.inf, s)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_mlp(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """down( SiLU(gate h) * (up h) ).  "Failed Star / fs" block figure ("SwiGLU → down")."""
    return (silu(h @ w_gate.T) * (h @ w_up.T)) @ w_down.T


def argmax_lowest(logits: np.ndarray) -> int:
    """Greedy choice: index of the largest logit, ties broken toward the lowest index."""
    return int(np.argmax(logits))


class KVCache:
    """Per-layer keys (after RoPE) and values for positions 0..length-1, float64."""

    def __init__(self, n_layers: int, n_kv: int, d: int, capacity: int):
        self.k = [np.zeros((capacity, n_kv, d)) for _ in range(n_layers)]
        self.v = [np.zeros((capacity, n_kv, d)) for _ in range(n_layers)]
        self.capacity = capacity
        self.length = 0


class OracleModel:
    """The whole decoder as its plain definition.

    ``forward(tokens, cache)`` runs the new tokens at positions
    cache.length .. cache.length+n-1 through every layer and returns the logits
    of every new row.  With an empty cache this is the cacheless forward over
    the whole prefix (the plain, cache-free definition); with a cache it is
    the same computation restricted to the new rows, because no earlier row
    depends on a later one.
    """

    def __init__(self, shape, weights: Dict, lora: Optional[List[Dict]] = None, lora_alpha: float = 0.0,
                 kv_bf16: bool = False):
        self.shape = shape
        # kv_bf16: the cache keeps keys (after RoPE) and values rounded to bf16,
        # and attention reads them back from it (the current rows included)
        self.kv_store = round_bf16 if kv_bf16 else (lambda a: a)
        self.E = widen_bf16(weights["embed"])
        self.final_norm = widen_bf16(weights["final_norm"])
        self.layers = []
        for lw in weights["layers"]:
            layer = {}
            for name, bits in lw.items():
                if shape.weight_format == _W_INT4_G128 and name in _PROJ:
                    codes, scales = quantize_int4_g128(widen_bf16_f32(bits))
                    layer[name] = dequantize_int4_g128(codes, scales)
                elif shape.weight_format == _W_Q8_0 and name in _PROJ:
                    codes, scales = quantize_q8_0(widen_bf16_f32(bits))
                    layer[name] = dequantize_q8_0(codes, scales)
                else:
                    layer[name] = widen_bf16(bits)
            self.layers.append(layer)
        self.lora = None
        if lora is not None:
            rank = lora[0]["a_q"].shape[0]
            self.lora_scale = lora_alpha / rank
            self.lora = [{k: widen_bf16(v) for k, v in lw.items()} for lw in lora]

    def layer_rows(self, li: int, x: np.ndarray, rows) -> np.ndarray:
        """Layer ``li`` applied to a prefix of rows, output only for ``rows``.

        x [n, H] holds the layer's input for positions 0..n-1 (a prompt from an
        empty cache).  Keys and values are formed for every position (each row
        attends to all earlier ones); queries, attention, o_proj and the MLP
        only for the selected rows.  The arithmetic is that of ``forward``
        restricted to those rows ("Failed Star / fs" block figure), so a
        layer's output can be checked on sampled rows at full model size.
        """
        s = self.shape
        w = self.layers[li]
        x = np.asarray(x, dtype=np.float64)
        rows = np.asarray(rows, dtype=np.int64)
        n = x.shape[0]
        nq, nkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim
        pos = np.arange(n)
        h = rmsnorm(x, w["attn_norm"], s.rms_eps)
        k = h @ w["wk"].T
        v = h @ w["wv"].T
        hr = h[rows]
        q = hr @ w["wq"].T
        if s.qkv_bias:
            q = q + w["bq"]
            k = k + w["bk"]
            v = v + w["bv"]
        if self.lora is not None:
            lw = self.lora[li]
            q = q + self.lora_scale * ((hr @ lw["a_q"].T) @ lw["b_q"].T)
            v = v + self.lora_scale * ((h @ lw["a_v"].T) @ lw["b_v"].T)
        q = q.reshape(len(rows), nq, d)
        k = k.reshape(n, nkv, d)
        v = v.reshape(n, nkv, d)
        if s.qk_norm:
            q = rmsnorm(q, w["q_norm"], s.rms_eps)
            k = rmsnorm(k, w["k_norm"], s.rms_eps)
        q = rope_rotate(q, rows, s.rope_theta)
        k = self.kv_store(rope_rotate(k, pos, s.rope_theta))
        v = self.kv_store(v)
        o = causal_gqa_attention(q, k, v, rows)
        xr = x[rows] + o.reshape(len(rows), nq * d) @ w["wo"].T
        h2 = rmsnorm(xr, w["mlp_norm"], s.rms_eps)
        return xr + swiglu_mlp(h2, w["w_gate"], w["w_up"], w["w_down"])

    def new_cache(self, capacity: Optional[int] = None) -> KVCache:
        s = self.shape
        return KVCache(s.n_layers, s.n_kv_heads, s.head_dim, capacity or s.max_pos)

    def forward(self, tokens, cache: Optional[KVCache] = None, capture: Optional[Dict] = None,
                logits_rows: str = "all") -> np.ndarray:
        s = self.shape
        tokens = np.asarray(tokens, dtype=np.int64)
        n = tokens.shape[0]
        if cache is None:
            cache = self.new_cache(max(n, 1))
        p0 = cache.length
        if p0 + n > cache.capacity:
            raise ValueError("oracle cache capacity exceeded")
        pos = np.arange(p0, p0 + n)
        nq, nkv, d = s.n_q_heads, s.n_kv_heads, s.head_dim

        # Gather: each token selects its row of the embedding table (a row copy, no product).
        x = self.E[tokens].copy()
        if capture is not None:
            capture["embed"] = x.copy()
            capture["layer_out"] = []

        for li, w in enumerate(self.layers):
            h = rmsnorm(x, w["attn_norm"], s.rms_eps)
            q = h @ w["wq"].T
            k = h @ w["wk"].T
            v = h @ w["wv"].T
            if s.qkv_bias:
                q = q + w["bq"]
                k = k + w["bk"]
                v = v + w["bv"]
            if self.lora is not None:
                lw = self.lora[li]
                q = q + self.lora_scale * ((h @ lw["a_q"].T) @ lw["b_q"].T)
                v = v + self.lora_scale * ((h @ lw["a_v"].T) @ lw["b_v"].T)
            q = q.reshape(n, nq, d)
            k = k.reshape(n, nkv, d)
            v = v.reshape(n, nkv, d)
            if s.qk_norm:
                q = rmsnorm(q, w["q_norm"], s.rms_eps)
                k = rmsnorm(k, w["k_norm"], s.rms_eps)
            q = rope_rotate(q, pos, s.rope_theta)
            k = rope_rotate(k, pos, s.rope_theta)
            cache.k[li][p0:p0 + n] = self.kv_store(k)
            cache.v[li][p0:p0 + n] = self.kv_store(v)
            o = causal_gqa_attention(q, cache.k[li][:p0 + n], cache.v[li][:p0 + n], pos)
            x = x + o.reshape(n, nq * d) @ w["wo"].T
            h2 = rmsnorm(x, w["mlp_norm"], s.rms_eps)
            x = x + swiglu_mlp(h2, w["w_gate"], w["w_up"], w["w_down"])
            if capture is not None:
                capture["layer_out"].append(x.copy())
        cache.length = p0 + n

        xf = rmsnorm(x, self.final_norm, s.rms_eps)
        if capture is not None:
            capture["final_norm"] = xf.copy()
        if logits_rows == "last":
            xf = xf[-1:]
        # Tied head: the embedding table serves as the [V, H] output projection.
        logits = xf @ self.E.T
        if capture is not None:
            capture["logits"] = logits.copy()
        return logits
