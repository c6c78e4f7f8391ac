"""qd_sample_logits_static (static per-device scratch, no workspace) against
qd_sample_logits (caller's workspace) through the C ABI.

Both run the same kernels on the same seeded logits, so their tokens must be
equal exactly; each is also checked against the oracle's choice.  Two calls
in a row on the static entry point, the second over a smaller vocabulary and
top_k, show that the shared scratch's leftover contents from the first call
do not leak into the second; the largest call (512 slices, top_k 39) fills
nearly all of the array.
"""
import ctypes

import numpy as np
import pytest

import synth
from oracle import sample_top_k_top_p, uniform_for_step

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def both(torch, lib, qd, x_np, sampling, step):
    """(static token, workspace token) for one input, through the C ABI."""
    x = torch.from_numpy(x_np).cuda()
    t_static = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    t_ws = torch.full((1,), -2, dtype=torch.int32, device="cuda")
    sp = None if sampling is None else ctypes.byref(sampling)
    s = torch.cuda.current_stream()
    rc = lib.qd_sample_logits_static(x.data_ptr(), x_np.shape[0], sp, step, t_static.data_ptr(), s.cuda_stream)
    assert rc == 0, lib.qd_last_error(None)
    nb = lib.qd_sample_workspace_bytes(x_np.shape[0], sp)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    rc = lib.qd_sample_logits(x.data_ptr(), x_np.shape[0], sp, step, t_ws.data_ptr(), ws.data_ptr(), nb,
                              s.cuda_stream)
    assert rc == 0, lib.qd_last_error(None)
    s.synchronize()
    return int(t_static.item()), int(t_ws.item())


def oracle_choice(x_np, params, step):
    if params is None:
        return int(np.argmax(x_np.astype(np.float64)))
    T, k, p, seed = params
    return sample_top_k_top_p(x_np.astype(np.float64), T, k, p, uniform_for_step(seed, step))


@pytest.mark.parametrize("first,second", [
    ((524288, (1.0, 39, 1.0, 11)), (1000, (0.7, 8, 0.9, 12))),
    ((151936, (0.7, 40, 0.9, 13)), (4097, None)),
    ((151936, None), (63, (1.1, 63, 0.95, 14))),
])
def test_static_scratch_matches_workspace_entry_point(torch_cuda, first, second):
    import decoder_only_token_amd as qd
    lib = qd.load_library()
    for call, (vocab, params) in enumerate((first, second)):
        log(f"no-alloc sampler call {call}: V={vocab} params={params}")
        sp = None if params is None else qd.make_sampling(*params)
        for step in range(3):
            x = synth.make_logits(vocab, 500 + 10 * call + step, scale=1.5, step=0.25 if step == 2 else None)
            got_static, got_ws = both(torch_cuda, lib, qd, x, sp, step)
            assert got_static == got_ws, (vocab, params, step, got_static, got_ws)
            want = oracle_choice(x, params, step)
            if got_static != want:
                T, k, p, seed = params
                u = uniform_for_step(seed, step)
                assert any(sample_top_k_top_p(x.astype(np.float64), T, k, p, uu) == got_static
                           for uu in (max(0.0, u - 1e-5), min(1.0 - 1e-12, u + 1e-5))), (vocab, step)


def test_static_entry_point_rejects_bad_arguments(torch_cuda):
    import decoder_only_token_amd as qd
    lib = qd.load_library()
    x = torch_cuda.zeros(16, dtype=torch_cuda.float32, device="cuda")
    t = torch_cuda.zeros(1, dtype=torch_cuda.int32, device="cuda")
    assert lib.qd_sample_logits_static(x.data_ptr(), 524289, None, 0, t.data_ptr(), 0) == -1
    sp40 = qd.make_sampling(0.7, 40, 0.9, 1)  # 513 * 40 > 20480
    assert lib.qd_sample_logits_static(x.data_ptr(), 524288, ctypes.byref(sp40), 0, t.data_ptr(), 0) == -1
    sp = qd.make_sampling(0.7, 17, 0.9, 1)
    assert lib.qd_sample_logits_static(x.data_ptr(), 16, ctypes.byref(sp), 0, t.data_ptr(), 0) == -1
    assert lib.qd_sample_logits_static(None, 16, None, 0, t.data_ptr(), 0) == -1
