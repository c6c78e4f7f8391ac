"""GPU parity: the HIP library against the float64 oracle on seeded inputs.

Bar: every logit within |got - want| <= 2e-3 + 2e-3 |want|, and the GPU's
greedy token equal to the oracle's argmax except at near-ties (two candidates
within that tolerance on the oracle's logits), which are counted and must stay rare.
"""
import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import OracleModel

from gpu_util import lockstep_greedy, logits_within_tol, near_tie, sampling_mismatch_explained, to_device

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


PATHS = {"persistent": 0, "graph": 1}


def make_decoder(torch_cuda, shape, max_prefill, lora_rank_max=0, path="persistent"):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max, decode_path=PATHS[path])
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


def assert_records(recs, max_forced=0):
    bad = [r for r in recs if r.n_bad]
    assert not bad, f"logits out of tolerance at steps {[(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]}"
    forced = [r for r in recs if r.forced]
    assert len(forced) <= max_forced, f"token mismatches (near-ties) at {[(r.step, r.gpu_token, r.oracle_token) for r in forced]}"


@pytest.mark.parametrize("path", ["persistent", "graph"])
@pytest.mark.parametrize("random_gains", [False, True])
def test_tiny_prefill_and_decode(torch_cuda, random_gains, path):
    """8-token prompt then 16 greedy steps on the 2-layer tiny model; every step checked."""
    wl = synth.WORKLOADS["tiny"]
    shape = wl.shape
    log(f"tiny random_gains={random_gains} path={path}")
    w = synth.make_weights(shape, random_gains=random_gains)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, wl.max_prefill, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    recs = lockstep_greedy(dec, oracle, prompt, wl.decode_steps, log=log)
    assert_records(recs)


def test_tiny_capture_checkpoints(torch_cuda):
    """Embedding, every layer's output, final norm and logits of a 13-token prefill."""
    import decoder_only_token_amd as qd
    shape = synth.TINY
    w = synth.make_weights(shape, seed=5, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, 13, seed=6)
    dec.prefill(prompt)
    cap = {}
    oracle.forward(prompt, capture=cap)
    H = shape.hidden
    got = dec.get_capture(qd.QD_CAP_EMBED, 0, 13 * H).reshape(13, H)
    assert np.array_equal(got, cap["embed"].astype(np.float32))
    for l in range(shape.n_layers):
        got = dec.get_capture(qd.QD_CAP_LAYER_OUT, l, 13 * H).reshape(13, H)
        np.testing.assert_allclose(got, cap["layer_out"][l], rtol=1e-3, atol=1e-3)
    got = dec.get_capture(qd.QD_CAP_FINAL_NORM, 0, H)
    np.testing.assert_allclose(got, cap["final_norm"][-1], rtol=1e-3, atol=1e-3)
    got = dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab)
    ok, ratio, nbad = logits_within_tol(got, cap["logits"][-1])
    assert ok, (ratio, nbad)
    with pytest.raises(qd.QdError):
        dec.get_capture(qd.QD_CAP_LOGITS, 0, shape.vocab - 1)  # capacity too small


def test_tiny_errors_leave_state_unchanged(torch_cuda):
    import decoder_only_token_amd as qd
    shape = synth.TINY
    dec = make_decoder(torch_cuda, shape, 16)
    with pytest.raises(qd.QdError) as e:
        dec.prefill([1, 2, 3])
    assert e.value.code == -3  # no weights
    w = synth.make_weights(shape, seed=7)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    with pytest.raises(qd.QdError) as e:
        dec.decode_step()
    assert e.value.code == -3  # decode before prefill
    with pytest.raises(qd.QdError) as e:
        dec.prefill([])
    assert e.value.code == -1
    with pytest.raises(qd.QdError) as e:
        dec.prefill(list(range(17)))
    assert e.value.code == -4  # > max_prefill
    with pytest.raises(qd.QdError) as e:
        dec.prefill([shape.vocab])
    assert e.value.code == -1
    assert dec.position == 0
    dec.prefill([1, 2])
    assert dec.position == 2


@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_tiny_runs_are_bit_identical(torch_cuda, path):
    import torch
    shape = synth.TINY
    w = synth.make_weights(shape, seed=8)
    dec = make_decoder(torch_cuda, shape, 16, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    outs = []
    for _ in range(2):
        logits = torch.empty((6, shape.vocab), dtype=torch.float32, device="cuda")
        dec.reset_kv()
        dec.prefill([5, 6, 7, 8], logits_out=logits[0])
        for i in range(1, 6):
            dec.decode_step(logits_out=logits[i])
        torch.cuda.synchronize()
        outs.append(logits.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_tiny_prefill_equals_sequential_decode(torch_cuda):
    """Batched prefill of 12 tokens vs 1-token prefill + forced 1-token appends: logits agree."""
    import torch
    shape = synth.TINY
    w = synth.make_weights(shape, seed=9)
    dec = make_decoder(torch_cuda, shape, 16)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    toks = synth.make_prompt(shape.vocab, 12, seed=10)
    a = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    b = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    dec.prefill(toks, logits_out=a)
    dec.reset_kv()
    for t in toks:
        dec.prefill([t], logits_out=b)
    torch.cuda.synchronize()
    np.testing.assert_allclose(a.cpu().numpy(), b.cpu().numpy(), rtol=1e-4, atol=1e-4)


@pytest.mark.slow
@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_qwen3_06b_prompt5_decode128(torch_cuda, path):
    """The Qwen3-0.6B-shaped workload: 5-token prompt, 128 greedy decode steps, every step checked."""
    wl = synth.WORKLOADS["qwen3-0.6b"]
    shape = wl.shape
    log(f"qwen3-0.6b path={path}: drawing weights")
    w = synth.make_weights(shape)
    dec = make_decoder(torch_cuda, shape, wl.max_prefill, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    log("qwen3-0.6b: building oracle")
    oracle = OracleModel(shape, w)
    del w
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    recs = lockstep_greedy(dec, oracle, prompt, wl.decode_steps, log=log)
    assert_records(recs, max_forced=2)


@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_tiny_sampling_topk_topp(torch_cuda, path):
    """T = 0.7, top-k 40, top-p 0.9 with a fixed seed on the tiny model, 24 steps.

    Every step: logits within tolerance, and the drawn token equal to the
    oracle's draw with the same uniform, except where the draw sits within
    1e-3 of a CDF boundary or the token is at the top-k cut (then the oracle's
    token is forced and the case is counted)."""
    import decoder_only_token_amd as qd
    shape = synth.TINY
    params = (0.7, 40, 0.9, 1234567)
    log(f"tiny sampling path={path}")
    w = synth.make_weights(shape, seed=11)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    sp = qd.make_sampling(*params)
    prompt = synth.make_prompt(shape.vocab, 8, seed=12)
    wants = {}

    def keep(msg):
        log(msg)

    recs = lockstep_greedy(dec, oracle, prompt, 24, sampling=sp, sampling_params=params, log=keep,
                           want_log=wants)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio) for r in bad]
    distinct = {r.oracle_token for r in recs}
    assert len(distinct) > 3, "sampling produced too few distinct tokens to exercise the draw"
    for r in recs:
        if r.forced:
            assert sampling_mismatch_explained(wants[r.step], params, r.step, r.gpu_token), \
                f"step {r.step}: gpu drew {r.gpu_token}, oracle {r.oracle_token}"
    assert sum(r.forced for r in recs) <= 2


@pytest.mark.parametrize("top_k", [1, 64])
def test_tiny_sampling_limits(torch_cuda, top_k):
    """top_k = 1 is greedy; a tiny top_p keeps only the best token (greedy too)."""
    import torch
    import decoder_only_token_amd as qd
    shape = synth.TINY
    w = synth.make_weights(shape, seed=13)
    dec = make_decoder(torch_cuda, shape, 16)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = [3, 1, 4, 1, 5]
    sp = qd.make_sampling(0.9, top_k, 1e-6, 99)
    toks = []
    for s in (None, sp):
        dec.reset_kv()
        out = torch.empty(1, dtype=torch.int32, device="cuda")
        seq = []
        dec.prefill(prompt, sampling=s, token_out=out)
        seq.append(dec.sync_token())
        for _ in range(6):
            dec.decode_step(sampling=s, token_out=out)
            seq.append(dec.sync_token())
        toks.append(seq)
    assert toks[0] == toks[1]


def test_sampling_argument_errors(torch_cuda):
    import decoder_only_token_amd as qd
    shape = synth.TINY
    dec = make_decoder(torch_cuda, shape, 16)
    w = synth.make_weights(shape, seed=14)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    for bad in (qd.make_sampling(0.7, 0, 0.9, 1), qd.make_sampling(0.7, 65, 0.9, 1),
                qd.make_sampling(0.7, 40, 0.0, 1), qd.make_sampling(0.7, 40, 1.5, 1),
                qd.make_sampling(float("inf"), 40, 0.9, 1), qd.make_sampling(float("nan"), 40, 0.9, 1)):
        with pytest.raises(qd.QdError) as e:
            dec.prefill([1, 2], sampling=bad)
        assert e.value.code == -1
    assert dec.position == 0


@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_tiny_long_context_splits(torch_cuda, path):
    """A 200-token prefill then 90 decode steps on the tiny model with a 512-position
    cache: the decode attention runs with 2 and then 3 position splits (the split
    boundary at 256 is crossed); logits checked every 10th step and the last."""
    import dataclasses
    shape = dataclasses.replace(synth.TINY, max_pos=512)
    log(f"tiny long context path={path}")
    w = synth.make_weights(shape, seed=21)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 256, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 200, seed=22)
    recs = lockstep_greedy(dec, oracle, prompt, 90, check_every=10, log=log)
    assert_records(recs, max_forced=1)


def test_tiny_persistent_split_beyond_lookahead(torch_cuda):
    """Decode past 1600 positions on a tiny model with 16 kv heads (one q head
    each): the CU budget caps the persistent step at 8 attention splits per kv
    head, so a split holds more positions (201) than the K/V rows a CU loads
    ahead (192) and the rest stream in further batches; every step checked."""
    import dataclasses
    shape = dataclasses.replace(synth.TINY, n_q_heads=16, n_kv_heads=16, max_pos=1664)
    log("tiny, 16 kv heads, 1600-token context, persistent")
    w = synth.make_weights(shape, seed=23)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 1600, path="persistent")
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 1600, seed=24)
    recs = lockstep_greedy(dec, oracle, prompt, 4, log=log)
    assert_records(recs, max_forced=1)


def test_tiny_persistent_row_segment_roles(torch_cuda):
    """A shape whose o_proj (4 q heads: 512 columns) and down projection (1408
    columns) do not form the matrix-core tiles, so those roles multiply on the
    row-segment path with f32 inputs (the down role unpacking the activation
    pairs to f32) while QKV and gate/up use the tiles; QKV bias on, no QK-norm.
    8-token prompt, 16 greedy steps, every step checked."""
    import dataclasses
    shape = dataclasses.replace(synth.TINY, name="tiny-rowseg", n_q_heads=4, n_kv_heads=2, intermediate=1408,
                                qk_norm=False, qkv_bias=True)
    log("tiny, row-segment o_proj and down roles, persistent")
    w = synth.make_weights(shape, seed=25, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16, path="persistent")
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 8, seed=26)
    recs = lockstep_greedy(dec, oracle, prompt, 16, log=log)
    assert_records(recs)


def test_tiny_persistent_300_steps_across_tag_wrap(torch_cuda):
    """300 persistent decode steps: the value-pair buffers (SwiGLU activations,
    attention output) carry only 8 bits of the step number in their tags, so
    the step count wraps past 256 here, and past 192 positions the attention
    splits in two.  The GPU's own greedy tokens are fed to the oracle as one
    sequence: every token must be the argmax of the oracle's logits at its
    step (near-ties allowed), and the last three steps' logits are checked."""
    import torch
    shape = dataclasses.replace(synth.TINY, max_pos=320)
    log("tiny, 300 persistent decode steps")
    w = synth.make_weights(shape, seed=27, random_gains=True)
    dec = make_decoder(torch_cuda, shape, 16, path="persistent")
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 8, seed=28)
    buf = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    dec.prefill(prompt, token_out=tok)
    torch.cuda.synchronize()
    toks = [int(tok.item())]
    last = []
    for step in range(300):
        dec.decode_step(logits_out=buf, token_out=tok)
        torch.cuda.synchronize()
        toks.append(int(tok.item()))
        if step >= 297:
            last.append(buf.cpu().numpy().astype(np.float64))
    seq = list(prompt) + toks[:-1]  # every token the GPU consumed, in order
    want = OracleModel(shape, w).forward(seq)  # one logits row per consumed token
    bad = [k for k, t in enumerate(toks) if not near_tie(want[len(prompt) - 1 + k], t)]
    assert not bad, f"tokens that are not their step's argmax at steps {bad[:8]}"
    for i, got in enumerate(last):
        ok, ratio, nbad = logits_within_tol(got, want[len(seq) - 3 + i])
        log(f"step {297 + i}: err/tol {ratio:.3f}")
        assert ok, (297 + i, ratio, nbad)


@pytest.mark.parametrize("n", [16, 137])
def test_tiny_batched_prefill_matrix_cores(torch_cuda, n):
    """Prefills of >= 16 rows run the projections on the matrix cores (bf16 hi/lo
    split of the inputs).  Every layer's output for every row, the final norm
    and the logits are checked against the oracle; 137 rows leave a ragged
    second row tile."""
    import dataclasses
    import decoder_only_token_amd as qd
    shape = dataclasses.replace(synth.TINY, max_pos=256)
    w = synth.make_weights(shape, seed=31, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 160)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    dec.enable_capture(True)
    prompt = synth.make_prompt(shape.vocab, n, seed=32)
    log(f"batched prefill n={n}")
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
    # the next token continues from the batched cache
    assert dec.sync_token() == int(np.argmax(cap["logits"][-1])) or \
        cap["logits"][-1][dec.sync_token()] >= np.max(cap["logits"][-1]) - 4e-3


@pytest.mark.parametrize("shape_name,chunks", [("TINY", (100, 137, 63, 1, 40)), ("TINY_INT4", (200, 17, 2, 150))])
def test_chunked_prefill_attention(torch_cuda, shape_name, chunks):
    """Prompts fed in several prefill calls: each call's rows attend to the cache
    of the earlier calls plus their own causal prefix (flash prefill tiles of
    32 positions; 64 query vectors per block).  The logits after every call
    are checked against the oracle."""
    import dataclasses
    import torch
    base = getattr(synth, shape_name)
    shape = dataclasses.replace(base, max_pos=512)
    log(f"chunked prefill {shape.name} {chunks}")
    w = synth.make_weights(shape, seed=71, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 256, path="graph")
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, sum(chunks), seed=72)
    cache = oracle.new_cache(sum(chunks) + 16)
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    dec.reset_kv()
    at = 0
    for n in chunks:
        dec.prefill(prompt[at:at + n], logits_out=logits)
        want = oracle.forward(prompt[at:at + n], cache, logits_rows="last")[-1]
        at += n
        torch.cuda.synchronize()
        ok, ratio, nbad = logits_within_tol(logits.cpu().numpy(), want)
        log(f"after {at} rows: err/tol {ratio:.3f}")
        assert ok, (at, ratio, nbad)
    assert dec.position == at


@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_tiny_eight_query_heads_per_kv_head(torch_cuda, path):
    """bf16 model of the 3B family's structure (16 q / 2 kv heads: 8 query
    heads per kv head, q/k/v bias, no QK-norm) at 2 layers: 8-token prompt,
    16 greedy steps, every step checked on both decode paths."""
    shape = dataclasses.replace(synth.TINY_INT4, name="tiny-g8-bf16", weight_format=synth.W_BF16)
    log(f"tiny G=8 bf16 path={path}")
    w = synth.make_weights(shape, seed=29, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16, path=path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, 8, seed=30)
    recs = lockstep_greedy(dec, oracle, prompt, 16, log=log)
    assert_records(recs, max_forced=1)
