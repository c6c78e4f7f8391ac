"""Helpers shared by the GPU parity tests: upload synthetic weights as torch
device tensors, and drive the HIP library and the oracle in lockstep.

The oracle always follows its own greedy (or sampled) trajectory.  The GPU
is checked against it at every step; when the GPU's choice differs only by a
near-tie (the two candidates' oracle logits within the logit tolerance), the
GPU is forced onto the oracle's token by appending it with qd_prefill, so the
comparison continues on the oracle's inputs.  No GPU value ever feeds the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

ATOL = 2e-3
RTOL = 2e-3


def to_device(weights: Dict, device="cuda") -> Dict:
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    return {"embed": t(weights["embed"]), "final_norm": t(weights["final_norm"]),
            "layers": [{k: t(v) for k, v in lw.items()} for lw in weights["layers"]]}


def lora_to_device(lora: List[Dict], device="cuda") -> List[Dict]:
    import torch
    return [{k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(device) for k, v in lw.items()}
            for lw in lora]


def logits_within_tol(got: np.ndarray, want: np.ndarray):
    err = np.abs(got.astype(np.float64) - want)
    bound = ATOL + RTOL * np.abs(want)
    bad = err > bound
    return (not bad.any()), float(np.max(err / bound)), int(np.count_nonzero(bad))


def near_tie(want: np.ndarray, tok: int) -> bool:
    m = float(np.max(want))
    return float(want[tok]) >= m - (ATOL + RTOL * abs(m))


@dataclasses.dataclass
class StepRecord:
    step: int
    gpu_token: int
    oracle_token: int
    max_err_ratio: float
    n_bad: int
    forced: bool


def lockstep_greedy(dec, oracle, prompt, steps: int, check_every: int = 1, sampling=None, sampling_params=None,
                    log=None, want_log: Optional[Dict] = None) -> List[StepRecord]:
    """Prefill `prompt`, then `steps` decode steps, comparing every checked step."""
    import torch
    from oracle import argmax_lowest, sample_top_k_top_p, uniform_for_step

    V = oracle.shape.vocab
    logits_dev = torch.empty(V, dtype=torch.float32, device="cuda")
    tok_dev = torch.empty(1, dtype=torch.int32, device="cuda")
    cache = oracle.new_cache(len(prompt) + steps + 1)
    dec.reset_kv()
    dec.prefill(prompt, sampling=sampling, logits_out=logits_dev, token_out=tok_dev)
    want = oracle.forward(prompt, cache, logits_rows="last")[-1]
    recs = []
    for step in range(steps + 1):
        torch.cuda.synchronize()
        got_tok = int(tok_dev.item())
        assert dec.sync_token() == got_tok  # also raises if a decode step was abandoned
        if sampling_params is None:
            o_tok = argmax_lowest(want)
        else:
            T, k, p, seed = sampling_params
            o_tok = sample_top_k_top_p(want, T, k, p, uniform_for_step(seed, step))
        if want_log is not None:
            want_log[step] = want
        ok, ratio, nbad = True, 0.0, 0
        if step % check_every == 0 or step == steps:
            got = logits_dev.cpu().numpy()
            ok, ratio, nbad = logits_within_tol(got, want)
        forced = got_tok != o_tok
        recs.append(StepRecord(step, got_tok, o_tok, ratio, nbad, forced))
        if log:
            log(f"step {step}: gpu {got_tok} oracle {o_tok} err/tol {ratio:.3f} bad {nbad}")
        if step == steps:
            break
        if forced:
            dec.prefill([o_tok], sampling=sampling, logits_out=logits_dev, token_out=tok_dev)
        else:
            dec.decode_step(sampling=sampling, logits_out=logits_dev, token_out=tok_dev)
        want = oracle.forward([o_tok], cache, logits_rows="last")[-1]
    return recs


def sampling_mismatch_explained(want: np.ndarray, params, step: int, got_tok: int, delta: float = 1e-3) -> bool:
    """Whether a sampled token that differs from the oracle's is still a correct draw.

    The GPU draws from its own f32 logits, which may differ from the oracle's
    within the logit tolerance.  A different token is accepted when moving the
    uniform by at most `delta` (a CDF boundary between the two tokens), or
    moving the logits by at most the tolerance at the kept-set cut, gives it.
    """
    from oracle import sample_top_k_top_p, uniform_for_step
    T, k, p, seed = params
    u = uniform_for_step(seed, step)
    for uu in (max(0.0, u - delta), min(1.0 - 1e-12, u + delta)):
        if sample_top_k_top_p(want, T, k, p, uu) == got_tok:
            return True
    # a token at the edge of the kept set: its logit within tolerance of the
    # k-th largest, and the draw landing past the end of the kept set
    order = np.lexsort((np.arange(want.shape[0]), -want))
    kth = float(want[order[min(k, want.shape[0]) - 1]])
    tol = ATOL + RTOL * abs(kth)
    if abs(float(want[got_tok]) - kth) <= tol:
        return True
    return False
