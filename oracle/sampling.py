"""Oracle token selection: greedy argmax and temperature / top-k / top-p sampling.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"flashmoon demo/README.md — Qwen3-0.6B inference", Quick start and the
REPL command table: temp = 0 means greedy; otherwise temperature, top-k and
top-p shape the draw.  The page does not state the order or the tie rules, so
the plain reading is used:

  1. order the vocabulary by (logit descending, token id ascending) and keep
     the first top_k entries (top_k <= 0 keeps all);
  2. pi_i = exp((l_i - l_0) / T) / sum_j exp((l_j - l_0) / T) over the kept entries;
  3. keep the longest prefix whose mass *before* each entry is < top_p
     (so the entry that crosses top_p is kept; the first entry always is);
  4. Z = sum of the kept pi; pick the first i with u * Z < pi_0 + ... + pi_i.

The uniform u for a step is drawn by a counter-based generator: SplitMix64
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014).  The draw for step s (s = 0 is the token chosen after the prompt)
is the (s+1)-th output of SplitMix64 seeded with `seed`, and u is its top 24
bits divided by 2^24.
"""
from __future__ import annotations

import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64_output(seed: int, i: int) -> int:
    """The i-th output (i >= 1) of SplitMix64 started from state `seed`."""
    z = (seed + i * _GAMMA) & _MASK
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
    return z ^ (z >> 31)


def uniform_for_step(seed: int, step: int) -> float:
    return (splitmix64_output(seed, step + 1) >> 40) / float(1 << 24)


def sample_top_k_top_p(logits: np.ndarray, temperature: float, top_k: int, top_p: float, u: float) -> int:
    logits = np.asarray(logits, dtype=np.float64)
    v = logits.shape[0]
    if temperature <= 0.0 or top_k == 1:
        return int(np.argmax(logits))
    k = v if top_k <= 0 else min(top_k, v)
    order = np.lexsort((np.arange(v), -logits))[:k]
    l = logits[order]
    w = np.exp((l - l[0]) / temperature)
    pi = w / np.sum(w)
    before = np.concatenate([[0.0], np.cumsum(pi)[:-1]])
    keep = before < top_p
    keep[0] = True
    kept = pi[keep]
    z = np.sum(kept)
    c = np.cumsum(kept)
    idx = int(np.searchsorted(c, u * z, side="right"))
    idx = min(idx, kept.shape[0] - 1)
    return int(order[idx])
