"""The handle-free token choice (qd_sample_logits) against the oracle's.

Seeded f32 logits go to both sides unchanged.  Greedy choices are compared
exactly (the same f32 values are compared on both sides, ties to the lowest
id).  Draws use the oracle's uniform for the step; a different token is
accepted only when a move of the uniform by 1e-5 (the f32 weights' rounding
against the oracle's float64) gives it.  Sizes: one logit, fewer logits than
top_k's maximum, one partial slice, exact slice multiples with a ragged tail,
the 151,936-entry vocabulary, and the largest supported vocabulary (512
slices of 1024).
"""
import numpy as np
import pytest

import synth
from oracle import argmax_lowest, sample_top_k_top_p, uniform_for_step

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def choose(torch, logits_np, sampling, step):
    import decoder_only_token_amd as qd
    x = torch.from_numpy(logits_np).cuda()
    tok = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    nb = qd.sample_workspace_bytes(logits_np.shape[0], sampling)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    s = torch.cuda.current_stream()
    qd.sample_logits(x, sampling, step, tok, ws, s.cuda_stream)
    s.synchronize()
    return int(tok.item())


def explained(logits_np, params, step, got, delta=1e-5):
    T, k, p, seed = params
    u = uniform_for_step(seed, step)
    return any(sample_top_k_top_p(logits_np.astype(np.float64), T, k, p, uu) == got
               for uu in (max(0.0, u - delta), min(1.0 - 1e-12, u + delta)))


VOCABS = [1, 7, 63, 1000, 1024, 1025, 4109, 151936, 524288]


@pytest.mark.parametrize("vocab", VOCABS)
def test_greedy_matches_oracle_exactly(torch_cuda, vocab):
    import decoder_only_token_amd as qd
    log(f"handle-free greedy, V={vocab}")
    for seed, step in ((60, None), (61, 0.25)):  # continuous logits, then many ties
        x = synth.make_logits(vocab, seed, step=step)
        want = argmax_lowest(x.astype(np.float64))
        assert choose(torch_cuda, x, None, 0) == want
        assert choose(torch_cuda, x, qd.make_sampling(0.0, 0, 0.0, 5), 3) == want  # temperature 0 = greedy
        assert choose(torch_cuda, x, qd.make_sampling(0.8, 1, 0.9, 5), 3) == want  # top_k 1 = greedy


@pytest.mark.parametrize("vocab", VOCABS)
@pytest.mark.parametrize("params", [(0.7, 40, 0.9, 1234), (1.3, 64, 1.0, 99), (0.5, 5, 0.5, 7)])
def test_draws_match_oracle(torch_cuda, vocab, params):
    import decoder_only_token_amd as qd
    T, k, p, seed = params
    k = min(k, vocab, 20480 // (-(-vocab // 1024) + 1))  # the merge's LDS bound
    params = (T, k, p, seed)
    sp = qd.make_sampling(T, k, p, seed)
    log(f"handle-free draw, V={vocab}, params={params}")
    forced = 0
    distinct = set()
    for step in range(24):
        x = synth.make_logits(vocab, 70 + step, scale=1.5, step=0.25 if step % 3 == 2 else None)
        want = sample_top_k_top_p(x.astype(np.float64), T, k, p, uniform_for_step(seed, step))
        got = choose(torch_cuda, x, sp, step)
        distinct.add(want)
        if got != want:
            assert explained(x, params, step, got), f"step {step}: gpu {got}, oracle {want}"
            forced += 1
    assert forced <= 1
    if vocab >= 1000 and k >= 5:
        assert len(distinct) > 3


def test_workspace_reused_across_sizes_in_one_stream(torch_cuda):
    """One workspace, calls of shrinking vocabulary and top_k queued back to
    back on one stream, read once at the end: each call's lists overwrite
    the last call's before the merge reads them."""
    import decoder_only_token_amd as qd
    torch = torch_cuda
    params = (0.9, 32, 0.95, 4321)
    sp = qd.make_sampling(*params)
    sizes = [151936, 50000, 4096, 1025, 33]
    ws = torch.empty(qd.sample_workspace_bytes(sizes[0], sp), dtype=torch.uint8, device="cuda")
    toks = torch.full((len(sizes),), -1, dtype=torch.int32, device="cuda")
    xs = [synth.make_logits(v, 90 + i, scale=1.5) for i, v in enumerate(sizes)]
    s = torch.cuda.current_stream()
    dev = [torch.from_numpy(x).cuda() for x in xs]
    for i, x in enumerate(dev):
        qd.sample_logits(x, sp, i, toks[i:i + 1], ws, s.cuda_stream)
    s.synchronize()
    got = toks.cpu().numpy()
    for i, x in enumerate(xs):
        want = sample_top_k_top_p(x.astype(np.float64), *params[:3], uniform_for_step(params[3], i))
        assert got[i] == want or explained(x, params, i, int(got[i])), (sizes[i], got[i], want)


def test_device_errors_are_reported(torch_cuda):
    import decoder_only_token_amd as qd
    torch = torch_cuda
    x = torch.zeros(2000, dtype=torch.float32, device="cuda")
    tok = torch.zeros(1, dtype=torch.int32, device="cuda")
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(qd.QdError, match="workspace"):
        qd.sample_logits(x, qd.make_sampling(0.7, 40, 0.9, 1), 0, tok, small, 0)
