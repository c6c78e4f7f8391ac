"""GPU parity of the rank-r LoRA adapter on q_proj / v_proj against the float64
oracle, and the promise that clearing it gives the base model back bit for bit."""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel

from gpu_util import ATOL, RTOL, lockstep_greedy, logits_within_tol, lora_to_device, to_device

pytestmark = pytest.mark.gpu

RANK, ALPHA = 16, 32.0


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make_decoder(torch_cuda, shape, max_prefill, lora_rank_max=RANK, path="graph"):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max,
                         decode_path=qd.QD_DECODE_GRAPH if path == "graph" else qd.QD_DECODE_PERSISTENT)
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


SHAPES = {"bf16": dataclasses.replace(synth.TINY, max_pos=256), "int4": synth.TINY_INT4}


def run_logits(torch_cuda, dec, prompt, steps):
    """Logits (host f32) of the prefill and of `steps` greedy decode steps.  The
    handle runs on a stream of its own, so each read waits for the device."""
    V = dec.cfg.vocab
    out = []
    buf = torch_cuda.empty(V, dtype=torch_cuda.float32, device="cuda")
    dec.reset_kv()
    dec.prefill(prompt, logits_out=buf)
    torch_cuda.cuda.synchronize()
    out.append(buf.cpu().numpy().copy())
    for _ in range(steps):
        dec.decode_step(logits_out=buf)
        torch_cuda.cuda.synchronize()
        out.append(buf.cpu().numpy().copy())
    return out


@pytest.mark.parametrize("path", ["graph", "persistent"])
@pytest.mark.parametrize("fmt", ["bf16", "int4"])
def test_lora_decode_parity(torch_cuda, fmt, path):
    """8-token prompt and 12 greedy steps with a rank-16 adapter (alpha 32); the
    adapter moves the oracle's logits far beyond the tolerance, and the GPU
    follows the adapted oracle.  On the persistent step one more CU computes
    the adapter's down products and the attention items add the up products."""
    shape = SHAPES[fmt]
    log(f"lora decode {shape.name} path={path}")
    w = synth.make_weights(shape, seed=51, random_gains=True)
    lora = synth.make_lora(shape, RANK, seed=52)
    base = OracleModel(shape, w)
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=ALPHA)
    prompt = synth.make_prompt(shape.vocab, 8, seed=53)
    moved = np.max(np.abs(oracle.forward(prompt)[-1] - base.forward(prompt)[-1]))
    assert moved > 10 * (ATOL + RTOL), moved
    dec = make_decoder(torch_cuda, shape, 16, path=path)
    dw, dl = to_device(w), lora_to_device(lora)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.set_lora(dl, RANK, ALPHA)
    recs = lockstep_greedy(dec, oracle, prompt, 12, log=log)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]
    assert sum(r.forced for r in recs) == 0


@pytest.mark.parametrize("fmt,n", [("bf16", 37), ("int4", 70)])
def test_lora_batched_prefill(torch_cuda, fmt, n):
    """A prefill of >= 16 rows runs the adapter's down product on the matrix
    cores; every layer's output, the final norm and the logits are checked."""
    import decoder_only_token_amd as qd
    shape = SHAPES[fmt]
    log(f"lora batched prefill {shape.name} n={n}")
    w = synth.make_weights(shape, seed=54, random_gains=True)
    lora = synth.make_lora(shape, RANK, seed=55)
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=ALPHA)
    dec = make_decoder(torch_cuda, shape, 128)
    dw, dl = to_device(w), lora_to_device(lora)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.set_lora(dl, RANK, ALPHA)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, n, seed=56)
    dec.prefill(prompt)
    cap = {}
    oracle.forward(prompt, capture=cap)
    H = shape.hidden
    for l in range(shape.n_layers):
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, l, n * H).reshape(n, H)
        np.testing.assert_allclose(got, cap["layer_out"][l], rtol=1e-3, atol=1e-3)
    got = dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab)
    ok, ratio, nbad = logits_within_tol(got, cap["logits"][-1])
    assert ok, (ratio, nbad)


@pytest.mark.parametrize("path", ["graph", "persistent"])
@pytest.mark.parametrize("fmt", ["bf16", "int4"])
def test_lora_cleared_is_bit_exact_base(torch_cuda, fmt, path):
    """Base run; adapter set (outputs change); adapter cleared: the logits of
    every step equal the base run's bit for bit.  An adapter with B = 0 also
    leaves every logit unchanged: bit for bit on the graph path and in the
    prefill; on the persistent step, whose plan gives the adapter's down
    products a CU of their own (the other roles' rows are split otherwise, so
    their sums run in another order), within the logit tolerance."""
    import torch
    shape = SHAPES[fmt]
    log(f"lora cleared {shape.name} path={path}")
    w = synth.make_weights(shape, seed=57)
    lora = synth.make_lora(shape, RANK, seed=58)
    dec = make_decoder(torch_cuda, shape, 32, path=path)
    dw, dl = to_device(w), lora_to_device(lora)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompts = [synth.make_prompt(shape.vocab, 5, seed=59), synth.make_prompt(shape.vocab, 20, seed=60)]
    for prompt in prompts:  # 5 rows: GEMV prefill; 20 rows: matrix-core prefill
        base = run_logits(torch_cuda, dec, prompt, 6)
        dec.set_lora(dl, RANK, ALPHA)
        adapted = run_logits(torch_cuda, dec, prompt, 6)
        assert np.max(np.abs(adapted[0] - base[0])) > 1e-2
        dec.clear_lora()
        again = run_logits(torch_cuda, dec, prompt, 6)
        for i, (a, b) in enumerate(zip(base, again)):
            assert np.array_equal(a, b), (len(prompt), i, float(np.max(np.abs(a - b))))
        zero = [{**lw, "b_q": torch.zeros_like(lw["b_q"]), "b_v": torch.zeros_like(lw["b_v"])} for lw in dl]
        dec.set_lora(zero, RANK, ALPHA)
        zb = run_logits(torch_cuda, dec, prompt, 6)
        dec.clear_lora()
        for i, (a, b) in enumerate(zip(base, zb)):
            if path == "graph" or i == 0:
                assert np.array_equal(a, b), (len(prompt), i, float(np.max(np.abs(a - b))))
            else:  # the adapter's persistent step gives one CU to the down products: other row splits
                ok, ratio, nbad = logits_within_tol(a, b.astype(np.float64))
                assert ok, (len(prompt), i, ratio, nbad)


def test_lora_argument_errors(torch_cuda):
    import decoder_only_token_amd as qd
    shape = SHAPES["bf16"]
    w = synth.make_weights(shape, seed=61)
    dl = lora_to_device(synth.make_lora(shape, RANK, seed=62))
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    off = make_decoder(torch_cuda, shape, 16, lora_rank_max=0)
    off.load_weights(dw)
    with pytest.raises(qd.QdError) as e:
        off.set_lora(dl, RANK, ALPHA)
    assert e.value.code == -3
    dec = make_decoder(torch_cuda, shape, 16, lora_rank_max=8)
    dec.load_weights(dw)
    with pytest.raises(qd.QdError) as e:
        dec.set_lora(dl, RANK, ALPHA)  # rank 16 > lora_rank_max 8
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.set_lora(dl, 0, ALPHA)
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.set_lora(dl, 8, float("nan"))
    assert e.value.code == -1
    dec.clear_lora()  # clearing with nothing installed is fine
