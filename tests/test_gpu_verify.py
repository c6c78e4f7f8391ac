"""Speculative verification (qd_verify / qd_rewind) against the oracle.

qd_verify runs m tokens as one batch of rows and makes the greedy choice after
every row.  Every row's logits are compared with the oracle's (the same tokens
through its cache) and every choice must be the oracle's argmax or within the
logit tolerance of it.  Cases: both decode paths of the tiny model (the
projections as GEMVs over up to 8 rows), the tiny int4 model with 16 rows
(matrix-core projections, two passes of the multi-row LM head), one row, and
Q8_0 weights.  A greedy speculative loop (drafts taken from the oracle's
greedy continuation, some planted wrong) must produce the oracle's greedy
tokens, and a decode step after its rewinds must see exactly the accepted
prefix in the cache.  Past 512 cached positions the rows of a batch run the
split-K decode attention one by one (cases at 600-700 positions, with an
adapter and the bf16 cache).
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel, argmax_lowest

from gpu_util import logits_within_tol, near_tie, to_device

pytestmark = pytest.mark.gpu

TINY = dataclasses.replace(synth.TINY, max_pos=128)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make(torch, shape, path, max_prefill=32, lora_rank_max=0, kv_format=0):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max, kv_format=kv_format,
                         decode_path=None if path == "auto" else
                         (qd.QD_DECODE_PERSISTENT if path == "persistent" else qd.QD_DECODE_GRAPH))
    dec = qd.Decoder(cfg, torch.cuda.current_stream().cuda_stream)
    return dec


TINY_LONG = dataclasses.replace(synth.TINY, max_pos=1024)
INT4_LONG = dataclasses.replace(synth.TINY_INT4, max_pos=1024)

CASES = {
    # name: (shape, decode path, prompt length, m, adapter rank, bf16 cache)
    "tiny-graph-5": (TINY, "graph", 9, 5, 0, False),
    "tiny-persistent-8": (TINY, "persistent", 9, 8, 0, False),
    "tiny-int4-16": (synth.TINY_INT4, "graph", 7, 16, 0, False),
    "tiny-int4-1": (synth.TINY_INT4, "persistent", 7, 1, 0, False),
    "tiny-q8-6": (synth.TINY_Q8, "auto", 5, 6, 0, False),
    # past 512 cached positions each row runs the split-K decode attention
    "tiny-long-7": (TINY_LONG, "graph", 600, 7, 0, False),
    "int4-long-lora-bf16kv-9": (INT4_LONG, "graph", 700, 9, 8, True),
    "int4-long-persistent-16": (INT4_LONG, "persistent", 650, 16, 0, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_verify_rows_against_oracle(torch_cuda, case):
    import decoder_only_token_amd as qd
    from gpu_util import lora_to_device
    torch = torch_cuda
    shape, path, plen, m, rank, kv16 = CASES[case]
    log(f"verify {case}")
    w = synth.make_weights(shape, seed=61, random_gains=True)
    lora = synth.make_lora(shape, rank, seed=68) if rank else None
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=16.0, kv_bf16=kv16)
    dec = make(torch, shape, path, max_prefill=max(32, plen), lora_rank_max=rank,
               kv_format=qd.QD_KV_BF16 if kv16 else qd.QD_KV_F32)
    dw = to_device(w)
    torch.cuda.synchronize()
    dec.load_weights(dw)
    if lora:
        dec.set_lora(lora_to_device(lora), rank, 16.0)
    prompt = synth.make_prompt(shape.vocab, plen, seed=62)
    toks = synth.make_prompt(shape.vocab, m, seed=63)
    V = shape.vocab
    dec.reset_kv()
    dec.prefill(prompt)
    logits = torch.empty((m, V), dtype=torch.float32, device="cuda")
    choices = torch.full((m,), -1, dtype=torch.int32, device="cuda")
    dec.verify(toks, logits_out=logits, choices_out=choices)
    torch.cuda.synchronize()
    assert dec.position == plen + m
    got_l, got_c = logits.cpu().numpy(), choices.cpu().numpy()
    cache = oracle.new_cache(plen + m + 1)
    oracle.forward(prompt, cache, logits_rows="last")
    want = oracle.forward(toks, cache, logits_rows="all")
    for i in range(m):
        ok, ratio, nbad = logits_within_tol(got_l[i], want[i])
        assert ok, (i, ratio, nbad)
        assert near_tie(want[i], int(got_c[i])), (i, int(got_c[i]), argmax_lowest(want[i]))
    # the next input token is the last row's choice: a decode step continues from it
    nxt = torch.empty(V, dtype=torch.float32, device="cuda")
    dec.decode_step(logits_out=nxt)
    torch.cuda.synchronize()
    want_n = oracle.forward([int(got_c[-1])], cache, logits_rows="last")[-1]
    ok, ratio, nbad = logits_within_tol(nxt.cpu().numpy(), want_n)
    assert ok, (ratio, nbad)
    dec.close()


@pytest.mark.parametrize("path", ["graph", "persistent"])
def test_speculative_loop_gives_the_greedy_tokens(torch_cuda, path):
    """Greedy speculative decoding with drafts of 3 to 6 tokens taken from the
    oracle's greedy continuation, every other call one draft planted wrong:
    the produced tokens are greedy tokens of the oracle (teacher-forced on
    them), some calls accept several drafts and some reject, and a decode step
    afterwards matches the oracle on exactly the produced prefix."""
    import decoder_only_token_amd as qd
    torch = torch_cuda
    shape = TINY
    V = shape.vocab
    log(f"speculative loop path={path}")
    w = synth.make_weights(shape, seed=64, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make(torch, shape, path)
    dw = to_device(w)
    torch.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(V, 9, seed=65)
    # the oracle's greedy continuation (drafts come from it)
    cache = oracle.new_cache(128)
    want = oracle.forward(prompt, cache, logits_rows="last")[-1]
    seq = []
    for _ in range(48):
        t = argmax_lowest(want)
        seq.append(t)
        want = oracle.forward([t], cache, logits_rows="last")[-1]
    first = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.reset_kv()
    dec.prefill(prompt, token_out=first)
    torch.cuda.synchronize()
    produced = [int(first.item())]
    choices = torch.empty(qd.QD_VERIFY_MAX, dtype=torch.int32, device="cuda")
    accepts, calls = [], 0
    while len(produced) < 30:
        i = len(produced)
        k = 3 + calls % 4
        drafts = list(seq[i:i + k])
        if calls % 2 == 1 and k > 2:
            drafts[2] = (drafts[2] + 1) % V  # planted wrong: rejected from here on
        new = dec.speculative_step(produced[-1], drafts, choices)
        log(f"  call {calls}: at {len(produced)} drafts {drafts} -> {new}")
        accepts.append(len(new) - 1)
        produced += new
        calls += 1
    assert dec.position == len(prompt) + len(produced) - 1
    assert max(accepts) >= 3 and min(accepts) <= 2
    # teacher-forced: every produced token is a greedy choice of the oracle
    log(f"  seq      {seq[:32]}")
    log(f"  produced {produced}")
    cache = oracle.new_cache(128)
    want = oracle.forward(prompt, cache, logits_rows="last")[-1]
    for i, t in enumerate(produced):
        assert near_tie(want, t), (i, t, argmax_lowest(want))
        want = oracle.forward([t], cache, logits_rows="last")[-1]
    # the cache holds exactly prompt + produced[:-1]; one more step consumes produced[-1]
    out = torch.empty(V, dtype=torch.float32, device="cuda")
    dec.decode_step(logits_out=out)
    torch.cuda.synchronize()
    ok, ratio, nbad = logits_within_tol(out.cpu().numpy(), want)
    assert ok, (ratio, nbad)
    dec.close()


def test_verify_and_rewind_argument_errors(torch_cuda):
    import decoder_only_token_amd as qd
    torch = torch_cuda
    shape = dataclasses.replace(synth.TINY, max_pos=32)
    dec = make(torch, shape, "graph", max_prefill=20)
    dec.load_weights(to_device(synth.make_weights(shape, seed=66)))
    dec.reset_kv()
    dec.prefill(synth.make_prompt(shape.vocab, 10, seed=67))
    for bad, code in (([], -1), ([1] * 17, -1), ([shape.vocab], -1)):
        with pytest.raises(qd.QdError) as e:
            dec.verify(bad)
        assert e.value.code == code
    dec.verify([1] * 16)
    assert dec.position == 26
    with pytest.raises(qd.QdError) as e:
        dec.verify([1] * 7)  # 26 + 7 > 32
    assert e.value.code == -4
    with pytest.raises(qd.QdError) as e:
        dec.rewind(27, 1)
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.rewind(1, -1)
    assert e.value.code == -1
    dec.rewind(20, 5)
    assert dec.position == 6
    dec.decode_step()
    assert dec.position == 7
    dec.close()
