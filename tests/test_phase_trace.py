"""Host logic of the phase-trace summary on a synthetic stamp array: the
critical hops and compute times of a layer add up to its period, and the
hop floor is the smallest consumer hop."""
import dataclasses

import numpy as np

from decoder_only_token_amd.phase_trace import summarize


@dataclasses.dataclass
class _Shape:
    n_layers: int


def test_budget_telescopes_to_the_period():
    L, ncu = 6, 10
    role = [0, 0, 1, 2, 2, 3, 3, 3, 4, 4]
    rng = np.random.default_rng(5)
    tr = np.zeros((ncu, 8 * (5 * L + 2)), dtype=np.int64)
    t = 1000
    floor = 10 ** 9
    for l in range(L):
        for r in range(5):
            p = 5 * l + r
            ready_min = None
            for cu in range(ncu):
                if role[cu] != r:
                    continue
                hop = int(rng.integers(70, 150))
                floor = min(floor, hop) if 0 < l < L - 1 else floor
                tr[cu, 8 * p + 0] = t - 50
                tr[cu, 8 * p + 1] = t + hop
                tr[cu, 8 * p + 3] = t + hop + int(rng.integers(100, 300))
            t = max(tr[cu, 8 * p + 3] for cu in range(ncu) if role[cu] == r)
    out = summarize(_Shape(L), tr)
    period = float(out[-2].split("median ")[1].split(" us")[0])
    total = float(out[-2].split("= ")[1].split(" us")[0])
    # one layer's period equals its own critical hops + compute exactly; the
    # medians over layers can differ only by rounding to 0.01 us here since
    # each layer's sum is its period
    per_layer = []
    for l in range(1, L - 1):
        per_layer.append((max(tr[cu, 8 * (5 * l + 4) + 3] for cu in range(ncu) if role[cu] == 4)
                          - max(tr[cu, 8 * (5 * l - 1) + 3] for cu in range(ncu) if role[cu] == 4)) / 100)
    assert abs(period - np.median(per_layer)) < 1e-9
    assert total > 0
    rows = {line.split()[0]: line.split() for line in out[2:7]}
    assert abs(min(float(rows[k][6]) for k in rows) - floor / 100) < 1e-9
    assert out[0] == "CUs per role: qkv 2, attn 1, o_proj 2, gate_up 3, down 2"


def test_one_interior_layer_budget_is_exact():
    L, ncu = 3, 5
    tr = np.zeros((ncu, 8 * (5 * L + 2)), dtype=np.int64)
    t = 0
    for l in range(L):
        for r in range(5):
            p = 5 * l + r
            tr[r, 8 * p + 0] = t + 1
            tr[r, 8 * p + 1] = t + 100 + 10 * r
            tr[r, 8 * p + 3] = t + 300 + 7 * l
            t = tr[r, 8 * p + 3]
    out = summarize(_Shape(L), tr)
    period = float(out[-2].split("median ")[1].split(" us")[0])
    total = float(out[-2].split("= ")[1].split(" us")[0])
    assert abs(period - total) < 1e-9
    assert abs(period - 5 * 307 / 100) < 1e-9  # every phase of layer 1 publishes 307 ticks after the one before
