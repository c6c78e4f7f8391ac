"""GPU checks at the benchmark workloads' full sizes, in the launch
configuration bench.py times.

A full 28- or 36-layer float64 forward over thousands of rows is too slow for
a test, so the oracle checks outputs it can compute one by one: the output of
sampled layers on sampled rows, from the GPU's own input to that layer
(captured), and the whole LM head (final norm and every logit of the last row)
from the GPU's last hidden row.  The one-row step (the decode GEMVs and the
split-K decode attention over the whole cache) is checked the same way, layer
by layer, against the oracle's layer applied to the prompt's rows.  Where the
whole model is cheap enough (the 0.6B shape at 2042 positions), decode steps
are compared with the full oracle forward.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel, rmsnorm

from gpu_util import ATOL, RTOL, logits_within_tol, lora_to_device, to_device

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def weights_3b():
    log("drawing the 3B weights")
    return synth.make_weights(synth.QWEN25_3B_INT4)


def make_decoder(torch_cuda, shape, max_prefill, path, lora_rank_max=0):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max,
                         decode_path=qd.QD_DECODE_PERSISTENT if path == "persistent" else qd.QD_DECODE_GRAPH)
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


def one_layer_oracle(shape, w, li, lora=None, alpha=0.0):
    """Oracle holding only layer li (its weights widened / quantised as in the full model)."""
    s1 = dataclasses.replace(shape, n_layers=1)
    sub = {"embed": w["embed"][:1], "final_norm": w["final_norm"], "layers": [w["layers"][li]]}
    return OracleModel(s1, sub, lora=[lora[li]] if lora else None, lora_alpha=alpha)


def check_sampled(dec, shape, w, prompt, layers, rows, lora=None, alpha=0.0, tol=1e-3):
    import decoder_only_token_amd as qd
    n, H = len(prompt), shape.hidden
    for li in layers:
        x_in = (dec.get_capture(qd.QD_CAP_EMBED, 0, n * H) if li == 0
                else dec.get_capture(qd.QD_CAP_LAYER_OUT, li - 1, n * H)).reshape(n, H)
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, li, n * H).reshape(n, H)[rows]
        want = one_layer_oracle(shape, w, li, lora, alpha).layer_rows(0, x_in.astype(np.float64), rows)
        err = float(np.max(np.abs(got - want) / (tol + tol * np.abs(want))))
        log(f"layer {li} rows {list(rows)}: err/tol {err:.3f}")
        np.testing.assert_allclose(got, want, rtol=tol, atol=tol)
    # final norm and the whole tied head from the GPU's last hidden row
    x_last = dec.get_capture(qd.QD_CAP_LAYER_OUT, shape.n_layers - 1, n * H).reshape(n, H)[-1]
    g = synth.bf16_to_f32(w["final_norm"]).astype(np.float64)
    xf_want = rmsnorm(x_last.astype(np.float64), g, shape.rms_eps)
    xf = dec.get_capture(qd.QD_CAP_FINAL_NORM, 0, H)
    np.testing.assert_allclose(xf, xf_want, rtol=tol, atol=tol)
    E = synth.bf16_to_f32(w["embed"]).astype(np.float64)
    want = E @ xf.astype(np.float64)
    got = dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab)
    ok, ratio, nbad = logits_within_tol(got, want)
    log(f"LM head over {shape.vocab} rows: err/tol {ratio:.3f}")
    assert ok, (ratio, nbad)
    return got


def one_row_step_layers(dec, shape, w, prompt, layers, lora=None, alpha=0.0, tol=1e-3):
    """Prefill all but the last token, then the last one alone: the one-row
    kernels (decode GEMVs, split-K decode attention over the whole cache).
    Sampled layers of that row are checked against the oracle's layer applied
    to every row of the prompt (the earlier rows' inputs captured from the
    batched prefill, the last row's from the one-row step), and the LM head
    against the oracle from the step's last hidden row."""
    import decoder_only_token_amd as qd
    n, H = len(prompt), shape.hidden
    dec.reset_kv()
    dec.enable_capture(True)
    dec.prefill(prompt[:-1])
    ins = {li: (dec.get_capture(qd.QD_CAP_EMBED, 0, (n - 1) * H) if li == 0
                else dec.get_capture(qd.QD_CAP_LAYER_OUT, li - 1, (n - 1) * H)).reshape(n - 1, H)
           for li in layers}
    dec.prefill(prompt[-1:])
    for li in layers:
        last_in = (dec.get_capture(qd.QD_CAP_EMBED, 0, H) if li == 0
                   else dec.get_capture(qd.QD_CAP_LAYER_OUT, li - 1, H)).reshape(1, H)
        x_in = np.concatenate([ins[li], last_in]).astype(np.float64)
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, li, H)
        want = one_layer_oracle(shape, w, li, lora, alpha).layer_rows(0, x_in, [n - 1])[0]
        err = float(np.max(np.abs(got - want) / (tol + tol * np.abs(want))))
        log(f"one-row step at position {n - 1}, layer {li}: err/tol {err:.3f}")
        np.testing.assert_allclose(got, want, rtol=tol, atol=tol)
    x_last = dec.get_capture(qd.QD_CAP_LAYER_OUT, shape.n_layers - 1, H)
    g = synth.bf16_to_f32(w["final_norm"]).astype(np.float64)
    xf = dec.get_capture(qd.QD_CAP_FINAL_NORM, 0, H)
    np.testing.assert_allclose(xf, rmsnorm(x_last.astype(np.float64), g, shape.rms_eps), rtol=tol, atol=tol)
    E = synth.bf16_to_f32(w["embed"]).astype(np.float64)
    ok, ratio, nbad = logits_within_tol(dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab), E @ xf.astype(np.float64))
    log(f"one-row step LM head: err/tol {ratio:.3f}")
    assert ok, (ratio, nbad)
    dec.enable_capture(False)


def test_full_size_qwen3_06b_long_prefill_and_decode(torch_cuda):
    """qwen3-0.6b-long: 512-token batched prefill (matrix cores), sampled layers
    and the full LM head against the oracle; the one-row step layer by layer;
    then the cache is filled to 2040 positions and two persistent decode steps
    are compared with the whole oracle forward."""
    import torch
    wl = synth.WORKLOADS["qwen3-0.6b-long"]
    shape = wl.shape
    w = synth.make_weights(shape)
    dw = to_device(w)
    torch.cuda.synchronize()
    dec = make_decoder(torch_cuda, shape, wl.max_prefill, "persistent")
    dec.load_weights(dw)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    dec.prefill(prompt)
    check_sampled(dec, shape, w, prompt, layers=[0, 13, 27], rows=[0, 1, 255, 510, 511])
    dec.enable_capture(False)
    one_row_step_layers(dec, shape, w, prompt, layers=[0, 13, 27])
    # fill the cache to 2040 positions, then two persistent decode steps
    # (positions 2040 and 2041: 11 attention splits per kv head), compared
    # with the whole oracle forward over the same 2042 tokens
    from oracle import argmax_lowest
    chunks = [synth.make_prompt(shape.vocab, 512, seed=90 + i) for i in range(3)]
    chunks.append(synth.make_prompt(shape.vocab, 504, seed=93))
    dec.reset_kv()
    for ch in chunks:
        dec.prefill(ch)
    assert dec.position == 2040
    g0 = dec.sync_token()
    a = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    dec.decode_step(logits_out=a)  # consumes g0 at position 2040
    t1 = dec.sync_token()
    dec.decode_step(logits_out=b)  # consumes t1 at position 2041
    torch.cuda.synchronize()
    log("oracle forward over 2042 positions")
    oracle = OracleModel(shape, w)
    cache = oracle.new_cache(2048)
    fill = np.concatenate(chunks)
    w_fill = oracle.forward(fill, cache, logits_rows="last")[-1]
    w0 = oracle.forward([g0], cache, logits_rows="last")[-1]
    w1 = oracle.forward([t1], cache, logits_rows="last")[-1]
    for name, tok, want in (("prefill token", g0, w_fill), ("decode at 2040", t1, w0)):
        m = float(np.max(want))
        assert want[tok] >= m - (ATOL + RTOL * abs(m)), f"{name}: token {tok} is not the oracle's argmax {argmax_lowest(want)}"
    for pos, got, want in ((2040, a, w0), (2041, b, w1)):
        ok, ratio, nbad = logits_within_tol(got.cpu().numpy(), want)
        log(f"persistent decode at position {pos} vs oracle: err/tol {ratio:.3f}")
        assert ok, (pos, ratio, nbad)


def test_full_size_qwen25_3b_int4(torch_cuda, weights_3b):
    """qwen2.5-3b-int4 at full size (36 layers, int4 g128): the 256-token
    batched prefill on sampled layers and rows and the full LM head against
    the oracle, then the one-row step at position 255 layer by layer."""
    import torch
    wl = synth.WORKLOADS["qwen2.5-3b-int4"]
    shape = wl.shape
    w = weights_3b
    dw = to_device(w)
    torch.cuda.synchronize()
    dec = make_decoder(torch_cuda, shape, wl.max_prefill, "graph")
    dec.load_weights(dw)
    del dw
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    dec.prefill(prompt)
    check_sampled(dec, shape, w, prompt, layers=[0, 17, 35], rows=[0, 1, 100, 254, 255])
    dec.enable_capture(False)
    one_row_step_layers(dec, shape, w, prompt, layers=[0, 17, 35])


def test_full_size_qwen25_3b_int4_lora_8192(torch_cuda, weights_3b):
    """qwen2.5-3b-int4-lora at full size: rank-16 adapter (alpha 32), an
    8192-token batched prefill checked on sampled layers and rows and the full
    LM head; the one-row step at position 8191 layer by layer; and the
    cleared adapter giving the base model's logits bit for bit."""
    import torch
    wl = synth.WORKLOADS["qwen2.5-3b-int4-lora"]
    shape = wl.shape
    w = weights_3b
    lora = synth.make_lora(shape, wl.lora_rank)
    dw, dl = to_device(w), lora_to_device(lora)
    torch.cuda.synchronize()
    dec = make_decoder(torch_cuda, shape, wl.max_prefill, "graph", lora_rank_max=wl.lora_rank)
    dec.load_weights(dw)
    del dw
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    buf = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    dec.prefill(prompt[:512], logits_out=buf)
    torch.cuda.synchronize()
    base = buf.cpu().numpy().copy()
    dec.set_lora(dl, wl.lora_rank, wl.lora_alpha)
    dec.enable_capture(True)
    dec.reset_kv()
    dec.prefill(prompt)
    check_sampled(dec, shape, w, prompt, layers=[0, 35], rows=[0, 4095, 8190, 8191],
                         lora=lora, alpha=wl.lora_alpha)
    dec.enable_capture(False)
    one_row_step_layers(dec, shape, w, prompt, layers=[0, 35], lora=lora, alpha=wl.lora_alpha)
    dec.clear_lora()
    dec.reset_kv()
    dec.prefill(prompt[:512], logits_out=buf)
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), base)
