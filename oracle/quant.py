"""Oracle weight encodings: int4 group-128 and Q8_0 (int8 blocks of 32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"EMBERGLASS (qwen-webgpu-lora) README", sections "Why it's hard" and "Note on
weights": weights are quantised to symmetric int4 in groups of 128 on their
way to the GPU.  The page gives no formula, so the plainest symmetric reading
is used, with every rounding decision taken in float32 (the precision the GPU
quantiser uses, so both sides decide each code identically):

  for each output row n and each group of 128 consecutive input columns:
    s    = fp16_round_to_nearest_even( absmax(w_group) / 7 )   (f32 divide)
    code = round_half_even( w / float32(s) )                   (f32 divide)
           (s == 0  ->  every code is 0); codes lie in [-7, 7]
  the model's weight is code * s (exact in float32).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def quantize_int4_g128(w32: np.ndarray):
    """float32 [N, K] (K a multiple of 128) -> (codes int8 [N, K], scales float16 [N, K/128])."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    n, k = w32.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 128")
    g = w32.reshape(n, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    scales = (amax / np.float32(7.0)).astype(np.float16)
    s32 = scales.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(g / np.where(s32 > 0, s32, np.float32(1.0))), np.float32(0.0))
    q = np.clip(q, -7, 7).astype(np.int8)
    return q.reshape(n, k), scales


def dequantize_int4_g128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [N, K] and scales float16 [N, K/128] -> float64 [N, K] = code * scale."""
    s = np.repeat(scales.astype(np.float64), GROUP, axis=1)
    return codes.astype(np.float64) * s


# ---------------------------------------------------------------------------
# Q8_0 block quantisation: "SuperKittens pull request #7", the commit that
# adds the Q8_0 weight dtype (ggml type 8) and its matvec: blocks of 32 int8
# values with one fp16 scale.  The page names the format but prints no
# formula; the plainest symmetric reading is used, decisions again in float32:
#
#   for each output row n and each block of 32 consecutive input columns:
#     d    = fp16_round_to_nearest_even( absmax(w_block) / 127 )   (f32 divide)
#     code = round_half_even( w / float32(d) ), clipped to [-127, 127]
#            (d == 0  ->  every code is 0)
#   the model's weight is code * d (exact in float32).
BLOCK_Q8 = 32


def quantize_q8_0(w32: np.ndarray):
    """float32 [N, K] (K a multiple of 32) -> (codes int8 [N, K], scales float16 [N, K/32])."""
    w32 = np.ascontiguousarray(w32, dtype=np.float32)
    n, k = w32.shape
    if k % BLOCK_Q8:
        raise ValueError("K must be a multiple of 32")
    b = w32.reshape(n, k // BLOCK_Q8, BLOCK_Q8)
    amax = np.max(np.abs(b), axis=2)
    scales = (amax / np.float32(127.0)).astype(np.float16)
    s32 = scales.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(b / np.where(s32 > 0, s32, np.float32(1.0))), np.float32(0.0))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(n, k), scales


def dequantize_q8_0(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8 [N, K] and scales float16 [N, K/32] -> float64 [N, K] = code * scale."""
    s = np.repeat(scales.astype(np.float64), BLOCK_Q8, axis=1)
    return codes.astype(np.float64) * s
