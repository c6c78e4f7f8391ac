"""The bf16 KV cache (kv_format QD_KV_BF16, graph decode path) against the
oracle with the same cache rounding: keys (after RoPE) and values rounded to
bf16 at the store and read back by attention, the new rows included.

Every logit of every step is compared with the bf16-cache oracle
(`OracleModel(..., kv_bf16=True)`); tokens follow the greedy near-tie rule.
Cases: the tiny bf16 model with a GEMV prefill (9 rows) and with a
matrix-core prefill (37 rows, the prefill attention reading the bf16 cache),
the tiny int4 model with the rank-16 adapter, and the 3B-width int4 model.
"""
import dataclasses

import pytest

import synth
from oracle import OracleModel

from gpu_util import lockstep_greedy, lora_to_device, to_device

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


TINY = dataclasses.replace(synth.TINY, max_pos=128)
INT4_3B_2L = dataclasses.replace(synth.QWEN25_3B_INT4, name="qwen2.5-3b-int4-2layer", n_layers=2, vocab=4096,
                                 max_pos=128)

CASES = {
    # name: (shape, prompt length, steps, lora rank)
    "tiny-gemv-prefill": (TINY, 9, 16, 0),
    "tiny-mfma-prefill": (TINY, 37, 12, 0),
    "tiny-int4-lora": (synth.TINY_INT4, 20, 12, 16),
    "3b-int4": (INT4_3B_2L, 8, 12, 0),
}


@pytest.mark.parametrize("case", list(CASES))
def test_bf16_kv_cache_against_oracle(torch_cuda, case):
    import decoder_only_token_amd as qd
    shape, plen, steps, rank = CASES[case]
    log(f"bf16 KV cache, {case}")
    w = synth.make_weights(shape, seed=91, random_gains=True)
    lora = synth.make_lora(shape, rank, seed=92) if rank else None
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=32.0, kv_bf16=True)
    cfg = qd.make_config(shape, max_prefill=64, lora_rank_max=rank, decode_path=qd.QD_DECODE_GRAPH,
                         kv_format=qd.QD_KV_BF16)
    dec = qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    if lora:
        dec.set_lora(lora_to_device(lora), rank, 32.0)
    prompt = synth.make_prompt(shape.vocab, plen, seed=93)
    recs = lockstep_greedy(dec, oracle, prompt, steps, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) <= 1
    dec.close()
