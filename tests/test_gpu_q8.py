"""GPU parity of the Q8_0 weight format (int8 blocks of 32 with an fp16 scale)
against the float64 oracle.

The GPU quantises the bf16 weights itself while loading them; its codes and
scales must equal the oracle's encoding byte for byte (edge blocks planted:
all zero, fp16-subnormal scale, ties to even, one large value among small
ones).  The forward pass with those weights (the Q8_0 GEMVs for decode and, on
tiles of up to 8 rows, for prefills) is then held to the same logit tolerance
and greedy-token rule as the other formats.  Shapes: the tiny Q8_0 model
(widths 1024 and 1408: one pass, and a pass plus a ragged rest), the wide one
(2048 / 2432, 8 q heads per kv head, q/k/v bias) also with a rank-16 adapter
and the bf16 cache, and the 3B widths (K = 11008: 11 passes, two batches of
8), 2 layers.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel
from oracle.quant import quantize_q8_0

from gpu_util import lockstep_greedy, lora_to_device, to_device

pytestmark = pytest.mark.gpu

PROJ = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
Q8_3B_2L = dataclasses.replace(synth.QWEN25_3B_INT4, name="qwen2.5-3b-q8_0-2layer", n_layers=2, vocab=4096,
                               max_pos=64, weight_format=synth.W_Q8_0)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make_decoder(torch_cuda, shape, max_prefill, lora_rank_max=0, kv_format=0):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max, kv_format=kv_format)
    assert cfg.decode_path == qd.QD_DECODE_GRAPH
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


def plant_edge_blocks(w):
    """Edge cases of the encoding in layer 0's wq (bf16 bit patterns): row 0
    block 0 all zero (scale 0); row 1 block 0 tiny (fp16-subnormal scale);
    row 2 block 0 with scale 0.0078125 = 1.0 / 127 rounded... taken exact:
    amax 127 * 2^-7, values at w / d = +-2.5, +-0.5, 1.5 (ties to even); row
    3 block 1 one large value among small ones."""
    wq = synth.bf16_to_f32(w["layers"][0]["wq"]).copy()
    wq[0, :32] = 0.0
    wq[1, :32] = np.float32(3e-7) * np.sign(wq[1, :32] + 1e-9)
    d = np.float32(2.0 ** -7)
    row = np.full(32, 0.5 * d, np.float32)  # w / d = 0.5 -> 0
    row[0] = 127 * d
    row[1:9] = [2.5 * d, -2.5 * d, 0.5 * d, -0.5 * d, 1.5 * d, -1.5 * d, 3.5 * d, -127 * d]
    wq[2, :32] = row
    wq[3, 32:64] = np.float32(0.001)
    wq[3, 40] = np.float32(0.9)
    w["layers"][0]["wq"] = synth.bf16_round(wq)
    return w


@pytest.mark.parametrize("shape_name", ["TINY_Q8", "TINY_Q8_WIDE"])
def test_q8_quantiser_matches_oracle_encoding(torch_cuda, shape_name):
    shape = getattr(synth, shape_name)
    log(f"Q8_0 quantiser {shape.name}")
    w = plant_edge_blocks(synth.make_weights(shape, seed=51))
    dec = make_decoder(torch_cuda, shape, 16)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    for l in range(shape.n_layers):
        for name in PROJ:
            bits = w["layers"][l][name]
            codes, scales = quantize_q8_0(synth.bf16_to_f32(bits))
            got_c, got_s = dec.get_quantized(l, name, bits.shape)
            assert np.array_equal(got_c, codes), f"codes differ in layer {l} {name}"
            assert np.array_equal(got_s.view(np.uint16), scales.view(np.uint16)), f"scales differ in layer {l} {name}"
    c, s = dec.get_quantized(0, "wq", w["layers"][0]["wq"].shape)
    assert not c[0, :32].any() and s[0, 0] == 0
    assert list(c[2, :9]) == [127, 2, -2, 0, 0, 2, -2, 4, -127] and s[2, 0] == np.float16(2.0 ** -7)
    assert c[3, 40] == 127 and np.all(np.abs(c[3, 32:64][np.arange(32) != 8]) <= 1)
    dec.close()


@pytest.mark.parametrize("shape_name,plen", [("TINY_Q8", 8), ("TINY_Q8", 37), ("TINY_Q8_WIDE", 8),
                                              ("Q8_3B_2L", 8)])
def test_q8_prefill_and_decode(torch_cuda, shape_name, plen):
    """Prompt of `plen` tokens (the Q8_0 GEMVs on tiles of up to 8 rows: one
    tile, or five with a ragged last one), then 16 greedy steps on the
    per-operation graph, every step checked."""
    shape = Q8_3B_2L if shape_name == "Q8_3B_2L" else getattr(synth, shape_name)
    log(f"Q8_0 decode {shape.name} prompt {plen}")
    w = synth.make_weights(shape, seed=52, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 40)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    del dw
    prompt = synth.make_prompt(shape.vocab, plen, seed=53)
    recs = lockstep_greedy(dec, oracle, prompt, 16, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) <= 1
    dec.close()


def test_q8_with_adapter_and_bf16_cache(torch_cuda):
    """The wide Q8_0 model with the rank-16 adapter (alpha 32) and the bf16 KV
    cache: 8-token prompt and 12 greedy steps against the oracle with the same
    adapter and cache rounding; clearing the adapter gives the base model's
    logits bit for bit."""
    import decoder_only_token_amd as qd
    torch = torch_cuda
    shape = synth.TINY_Q8_WIDE
    log("Q8_0 + LoRA + bf16 KV")
    w = synth.make_weights(shape, seed=54, random_gains=True)
    lora = synth.make_lora(shape, 16, seed=55)
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=32.0, kv_bf16=True)
    dec = make_decoder(torch, shape, 16, lora_rank_max=16, kv_format=qd.QD_KV_BF16)
    dw = to_device(w)
    torch.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 8, seed=56)
    # the base model's first logits, before any adapter
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    dec.reset_kv()
    dec.prefill(prompt, logits_out=logits)
    torch.cuda.synchronize()
    base = logits.cpu().numpy().copy()
    dec.set_lora(lora_to_device(lora), 16, 32.0)
    recs = lockstep_greedy(dec, oracle, prompt, 12, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) <= 1
    dec.clear_lora()
    dec.reset_kv()
    dec.prefill(prompt, logits_out=logits)
    torch.cuda.synchronize()
    assert np.array_equal(logits.cpu().numpy(), base)
    dec.close()
