"""Multi-step decode (qd_decode_steps): n tokens per call with the token
feedback on the device and one host synchronisation at the end.

Each case prefills a prompt and runs the same number of greedy steps twice:
once as one qd_decode_steps call, once as single qd_decode_step calls from
the same state.  The token sequences and the last step's logits must agree
bit for bit (on the persistent path one launch runs every step whose plan has
the same attention split count, with each step's splits cut as its own plan
would cut them).  The batch's tokens are then checked against the oracle,
teacher-forced on them: at every step the chosen token is the oracle's argmax
or within the logit tolerance of it, and the last step's logits are within
tolerance.  Cases: the tiny bf16 model (one launch; and a run across a split
count change at context 192), the tiny int4 model, the 3B-width int4 model,
with the rank-16 adapter, and the graph path.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel

from gpu_util import logits_within_tol, lora_to_device, near_tie, to_device

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


TINY = dataclasses.replace(synth.TINY, max_pos=512)
INT4_3B_2L = dataclasses.replace(synth.QWEN25_3B_INT4, name="qwen2.5-3b-int4-2layer", n_layers=2, vocab=4096,
                                 max_pos=256)

CASES = {
    # name: (shape, path, prompt length, steps, lora rank)
    "tiny-persistent": (TINY, "persistent", 9, 24, 0),
    "tiny-persistent-split-change": (TINY, "persistent", 180, 24, 0),
    "tiny-int4-persistent": (synth.TINY_INT4, "persistent", 7, 20, 0),
    "3b-int4-persistent": (INT4_3B_2L, "persistent", 8, 16, 0),
    "3b-int4-persistent-lora": (INT4_3B_2L, "persistent", 8, 16, 16),
    "tiny-graph": (TINY, "graph", 9, 12, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_multistep_equals_single_steps_and_oracle(torch_cuda, case):
    import decoder_only_token_amd as qd
    torch = torch_cuda
    shape, path, plen, n, rank = CASES[case]
    log(f"multi-step {case}: prompt {plen}, {n} steps")
    w = synth.make_weights(shape, seed=81, random_gains=True)
    lora = synth.make_lora(shape, rank, seed=82) if rank else None
    cfg = qd.make_config(shape, max_prefill=256, lora_rank_max=rank,
                         decode_path=qd.QD_DECODE_PERSISTENT if path == "persistent" else qd.QD_DECODE_GRAPH)
    dec = qd.Decoder(cfg, torch.cuda.current_stream().cuda_stream)
    dw = to_device(w)
    torch.cuda.synchronize()
    dec.load_weights(dw)
    if lora:
        dec.set_lora(lora_to_device(lora), rank, 32.0)
    prompt = synth.make_prompt(shape.vocab, plen, seed=83)
    V = shape.vocab

    # one call
    dec.reset_kv()
    dec.prefill(prompt)
    toks_b = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    logits_b = torch.empty(V, dtype=torch.float32, device="cuda")
    dec.decode_steps(n, logits_out=logits_b, tokens_out=toks_b)
    torch.cuda.synchronize()
    assert dec.position == plen + n
    toks_b, logits_b = toks_b.cpu().numpy().copy(), logits_b.cpu().numpy().copy()
    assert dec.sync_token() == int(toks_b[-1])

    # single steps from the same state
    dec.reset_kv()
    dec.prefill(prompt)
    one = torch.empty(1, dtype=torch.int32, device="cuda")
    logits_s = torch.empty(V, dtype=torch.float32, device="cuda")
    toks_s = []
    for _ in range(n):
        dec.decode_step(logits_out=logits_s, token_out=one)
        torch.cuda.synchronize()
        toks_s.append(int(one.item()))
    assert toks_b.tolist() == toks_s
    assert np.array_equal(logits_b, logits_s.cpu().numpy())

    # the oracle, teacher-forced on the batch's tokens: step i consumes
    # inputs[i] (the prefill's choice, then the batch's tokens) and chooses toks_b[i]
    first = _first_token(dec, torch, prompt)
    inputs = [first] + [int(t) for t in toks_b[:-1]]
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=32.0)
    cache = oracle.new_cache(plen + n + 1)
    want = oracle.forward(prompt, cache, logits_rows="last")[-1]
    assert near_tie(want, first)
    for i in range(n):
        want = oracle.forward([inputs[i]], cache, logits_rows="last")[-1]
        assert near_tie(want, int(toks_b[i])), (i, int(toks_b[i]), int(np.argmax(want)))
    ok, ratio, nbad = logits_within_tol(logits_b, want)
    assert ok, (ratio, nbad)
    dec.close()


def _first_token(dec, torch, prompt):
    """The token the prefill chose (the first step's input)."""
    dec.reset_kv()
    t = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill(prompt, token_out=t)
    torch.cuda.synchronize()
    return int(t.item())


def test_multistep_argument_errors(torch_cuda):
    import decoder_only_token_amd as qd
    torch = torch_cuda
    shape = dataclasses.replace(synth.TINY, max_pos=32)
    cfg = qd.make_config(shape, max_prefill=16)
    dec = qd.Decoder(cfg, torch.cuda.current_stream().cuda_stream)
    dec.load_weights(to_device(synth.make_weights(shape, seed=84)))
    with pytest.raises(qd.QdError) as e:
        dec.decode_steps(2)  # before any prefill
    assert e.value.code == -3
    dec.prefill(synth.make_prompt(shape.vocab, 10, seed=85))
    with pytest.raises(qd.QdError) as e:
        dec.decode_steps(0)
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.decode_steps(23)  # 10 + 23 > 32
    assert e.value.code == -4
    dec.decode_steps(22)
    assert dec.position == 32
    dec.close()
