"""GPU parity of the int4 group-128 weight format against the float64 oracle.

The GPU quantises the bf16 weights itself while loading them; its codes and
scales must equal the oracle's encoding byte for byte.  The forward pass with
those weights (decode and short prefills on the int4 GEMVs, longer prefills on
the matrix cores) is then held to the same logit tolerance and greedy-token
rule as the bf16 path.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel
from oracle.quant import quantize_int4_g128

from gpu_util import lockstep_greedy, logits_within_tol, to_device

pytestmark = pytest.mark.gpu

PROJ = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make_decoder(torch_cuda, shape, max_prefill, path="graph"):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill,
                         decode_path=qd.QD_DECODE_GRAPH if path == "graph" else qd.QD_DECODE_PERSISTENT)
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


def plant_edge_groups(w):
    """Edge cases of the encoding in layer 0's wq (bf16 bit patterns):
    row 0 group 0 all zero (scale 0); row 1 group 0 tiny (fp16-subnormal
    scale); row 2 group 0 with scale 0.25 exactly and values at w / s = +-2.5,
    +-0.5 and 1.5 (ties to even); row 3 group 1 one large value among small ones."""
    wq = synth.bf16_to_f32(w["layers"][0]["wq"]).copy()
    wq[0, :128] = 0.0
    wq[1, :128] = np.float32(3e-7) * np.sign(wq[1, :128] + 1e-9)
    s = np.float32(0.25)
    row = np.full(128, 0.125, np.float32)  # w / s = 0.5 -> 0
    row[0] = 7 * s
    row[1:9] = [2.5 * s, -2.5 * s, 0.5 * s, -0.5 * s, 1.5 * s, -1.5 * s, 3.5 * s, -7 * s]
    wq[2, :128] = row
    wq[3, 128:256] = np.float32(0.001)
    wq[3, 200] = np.float32(0.9)
    w["layers"][0]["wq"] = synth.bf16_round(wq)
    return w


@pytest.mark.parametrize("shape_name", ["TINY_INT4", "TINY_INT4_WIDE"])
def test_int4_quantiser_matches_oracle_encoding(torch_cuda, shape_name):
    shape = getattr(synth, shape_name)
    log(f"int4 quantiser {shape.name}")
    w = plant_edge_groups(synth.make_weights(shape, seed=41))
    dec = make_decoder(torch_cuda, shape, 16)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    for l in range(shape.n_layers):
        for name in PROJ:
            bits = w["layers"][l][name]
            codes, scales = quantize_int4_g128(synth.bf16_to_f32(bits))
            got_c, got_s = dec.get_quantized(l, name, bits.shape)
            assert np.array_equal(got_c, codes), f"codes differ in layer {l} {name}"
            assert np.array_equal(got_s.view(np.uint16), scales.view(np.uint16)), f"scales differ in layer {l} {name}"
    c, s = dec.get_quantized(0, "wq", w["layers"][0]["wq"].shape)
    assert not c[0, :128].any() and s[0, 0] == 0
    assert list(c[2, :9]) == [7, 2, -2, 0, 0, 2, -2, 4, -7] and s[2, 0] == np.float16(0.25)


@pytest.mark.parametrize("path", ["graph", "persistent"])
@pytest.mark.parametrize("shape_name", ["TINY_INT4", "TINY_INT4_WIDE"])
def test_tiny_int4_prefill_and_decode(torch_cuda, shape_name, path):
    """8-token prompt (int4 GEMVs, two row tiles), then 16 greedy steps, every
    step checked; the decode steps run as the per-operation graph or as the
    persistent kernel (int4 slots on the int8 matrix cores; the 1408-column
    down projection of TINY_INT4 leaves 3 of the 8 waves a second group)."""
    shape = getattr(synth, shape_name)
    log(f"int4 decode {shape.name} path={path}")
    w = synth.make_weights(shape, seed=42, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16, path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 8, seed=43)
    recs = lockstep_greedy(dec, oracle, prompt, 16, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) == 0


@pytest.mark.parametrize("shape_name,n", [("TINY_INT4", 16), ("TINY_INT4", 137), ("TINY_INT4_WIDE", 70)])
def test_tiny_int4_batched_prefill_matrix_cores(torch_cuda, shape_name, n):
    """Prefills of >= 16 rows multiply the int4 codes on the matrix cores with
    the group scales applied per 128 columns; every layer's output row, the
    final norm and the logits are checked, then 8 decode steps continue."""
    import decoder_only_token_amd as qd
    shape = getattr(synth, shape_name)
    log(f"int4 batched prefill {shape.name} n={n}")
    w = synth.make_weights(shape, seed=44, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 160)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, n, seed=45)
    dec.prefill(prompt)
    cap = {}
    oracle.forward(prompt, capture=cap)
    H = shape.hidden
    for l in range(shape.n_layers):
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, l, n * H).reshape(n, H)
        np.testing.assert_allclose(got, cap["layer_out"][l], rtol=1e-3, atol=1e-3)
    got = dec.get_capture(qd.QD_CAP_FINAL_NORM, 0, H)
    np.testing.assert_allclose(got, cap["final_norm"][-1], rtol=1e-3, atol=1e-3)
    got = dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab)
    ok, ratio, nbad = logits_within_tol(got, cap["logits"][-1])
    assert ok, (ratio, nbad)
    dec.enable_capture(False)
    recs = lockstep_greedy(dec, oracle, prompt, 8, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) <= 1


def test_int4_readback_errors(torch_cuda):
    import decoder_only_token_amd as qd
    shape = synth.TINY_INT4
    dec = make_decoder(torch_cuda, shape, 16)
    with pytest.raises(qd.QdError) as e:
        dec.get_quantized(0, "wq", (shape.n_q_heads * 128, shape.hidden))
    assert e.value.code == -3  # no weights yet
    w = synth.make_weights(shape, seed=46)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    with pytest.raises(qd.QdError) as e:
        dec.get_quantized(shape.n_layers, "wq", (shape.n_q_heads * 128, shape.hidden))
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.get_quantized(0, "wq", (shape.n_q_heads * 128 - 1, shape.hidden))  # capacity too small
    assert e.value.code == -1
    bf = make_decoder(torch_cuda, dataclasses.replace(shape, weight_format=synth.W_BF16), 16)
    with pytest.raises(qd.QdError) as e:
        bf.get_quantized(0, "wq", (shape.n_q_heads * 128, shape.hidden))
    assert e.value.code == -3


def test_int4_edge_groups_through_both_paths(torch_cuda):
    """Weights with an all-zero group (scale 0), an fp16-subnormal scale and
    round-half-even ties, through the matrix-core prefill (40 rows: zero
    scales keep the running rescale unchanged) and the GEMV decode."""
    import decoder_only_token_amd as qd
    shape = synth.TINY_INT4
    w = plant_edge_groups(synth.make_weights(shape, seed=47, random_gains=True))
    # a whole zero row group in a second matrix as well, first and last group
    wo = synth.bf16_to_f32(w["layers"][1]["wo"]).copy()
    wo[5, :128] = 0.0
    wo[6, -128:] = 0.0
    w["layers"][1]["wo"] = synth.bf16_round(wo)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 64)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, 40, seed=48)
    dec.prefill(prompt)
    cap = {}
    oracle.forward(prompt, capture=cap)
    H = shape.hidden
    for l in range(shape.n_layers):
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, l, 40 * H).reshape(40, H)
        np.testing.assert_allclose(got, cap["layer_out"][l], rtol=1e-3, atol=1e-3)
    dec.enable_capture(False)
    recs = lockstep_greedy(dec, oracle, prompt[:6], 6, log=log)
    assert not [r for r in recs if r.n_bad]
