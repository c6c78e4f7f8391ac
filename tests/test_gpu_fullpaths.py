"""Oracle parity on the code paths the full-size workloads take.

The full models are too large for a float64 oracle run per step, so each test
here builds a model small enough for the oracle that still drives the exact
kernel instantiation or launch branch that a full-size workload runs:

* top-k / top-p sampling over the real 151,936-entry vocabulary (every slice
  list of the final merge in use), on both decode paths;
* the persistent step's attention merge with 9 to 11 position splits, which
  the 0.6B long-context workload runs past 1536 positions;
* the 3B-width int4 model (hidden 2048, intermediate 11008, 16/2 heads), whose
  down projection runs the 8-pass int4 GEMV and whose decode step is the
  captured 3B-width graph, or the persistent step with int4 slots (also on
  64 CUs, where the slots stream in during each phase);
* the graph path's decode attention for 8 q heads per kv head with several
  64-position tiles per split (16 kv heads, ~2100 positions), f32 and bf16
  cache, with an adapter whose rank is not a multiple of 8.

Every logit of every step is compared with the oracle; tokens follow the
greedy / sampled near-tie rules of gpu_util.
"""
import dataclasses

import numpy as np
import pytest

import synth
from oracle import OracleModel

from gpu_util import lockstep_greedy, sampling_mismatch_explained, to_device

pytestmark = pytest.mark.gpu

PATHS = {"persistent": 0, "graph": 1}


def log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def make_decoder(torch_cuda, shape, max_prefill, path, lora_rank_max=0):
    import decoder_only_token_amd as qd
    cfg = qd.make_config(shape, max_prefill=max_prefill, lora_rank_max=lora_rank_max, decode_path=PATHS[path])
    return qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)


def assert_records(recs, max_forced=0):
    bad = [r for r in recs if r.n_bad]
    assert not bad, f"logits out of tolerance at steps {[(r.step, r.max_err_ratio, r.n_bad) for r in bad[:5]]}"
    forced = [r for r in recs if r.forced]
    assert len(forced) <= max_forced, f"near-tie mismatches at {[(r.step, r.gpu_token, r.oracle_token) for r in forced]}"


# the 0.6B shape cut to 2 layers: same vocabulary (151,936), hidden, heads and MLP
QWEN3_2L = dataclasses.replace(synth.QWEN3_06B, name="qwen3-0.6b-2layer", n_layers=2, max_pos=64)
# the 3B int4 shape cut to 2 layers and a 4096-entry vocabulary
QWEN25_INT4_2L = dataclasses.replace(synth.QWEN25_3B_INT4, name="qwen2.5-3b-int4-2layer", n_layers=2, vocab=4096,
                                     max_pos=64)


@pytest.mark.parametrize("path", ["persistent", "graph"])
def test_sampling_full_vocabulary(torch_cuda, path):
    """T 0.7 / top-k 40 / top-p 0.9 with a fixed seed over V = 151,936 (149
    slice lists, so the final merge runs every list of every lane), 2-layer
    0.6B-width model, 8-token prompt and 28 steps: every logit checked, every
    draw equal to the oracle's or explained by the near-boundary rule."""
    import decoder_only_token_amd as qd
    shape = QWEN3_2L
    params = (0.7, 40, 0.9, synth.SEED_SAMPLING)
    log(f"full-vocabulary sampling path={path}")
    w = synth.make_weights(shape, seed=41)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 16, path)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    del dw
    sp = qd.make_sampling(*params)
    prompt = synth.make_prompt(shape.vocab, 8, seed=42)
    wants = {}
    recs = lockstep_greedy(dec, oracle, prompt, 28, sampling=sp, sampling_params=params, log=log, want_log=wants)
    bad = [r for r in recs if r.n_bad]
    assert not bad, [(r.step, r.max_err_ratio) for r in bad]
    assert len({r.oracle_token for r in recs}) > 10, "too few distinct draws to exercise the sampler"
    for r in recs:
        if r.forced:
            assert sampling_mismatch_explained(wants[r.step], params, r.step, r.gpu_token), \
                f"step {r.step}: gpu drew {r.gpu_token}, oracle {r.oracle_token}"
    assert sum(r.forced for r in recs) <= 2
    dec.close()


@pytest.mark.parametrize("prompt_len,splits", [(1700, 9), (1930, 11)])
def test_persistent_attention_merge_beyond_eight_splits(torch_cuda, prompt_len, splits):
    """Tiny model (16 q / 8 kv heads) with a 2048-position cache, as the 0.6B
    long-context workload: past 1536 positions the persistent step splits each
    kv head's positions into ceil(ctx / 192) = 9 .. 11 parts, and the merge
    folds them in two batches of up to 8.  Prompt of `prompt_len` tokens (one
    batched prefill), then 12 persistent decode steps, every logit checked."""
    shape = dataclasses.replace(synth.TINY, max_pos=2048)
    ctx = prompt_len + 1
    assert -(-ctx // 192) == splits
    log(f"persistent merge, prompt {prompt_len}: {splits} splits per kv head")
    w = synth.make_weights(shape, seed=43, random_gains=True)
    oracle = OracleModel(shape, w)
    dec = make_decoder(torch_cuda, shape, 2048, "persistent")
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    prompt = synth.make_prompt(shape.vocab, prompt_len, seed=44)
    recs = lockstep_greedy(dec, oracle, prompt, 12, log=log)
    assert_records(recs, max_forced=1)
    dec.close()


@pytest.mark.parametrize("path", ["graph", "persistent", "persistent-64cu", "persistent-lora"])
def test_int4_3b_width_decode(torch_cuda, path, monkeypatch):
    """2-layer model at the 3B int4 widths (hidden 2048, intermediate 11008,
    16 q / 2 kv heads, q/k/v bias, no QK-norm, int4 group-128, V 4096): the
    down projection (K = 11008) runs the 8-pass int4 GEMV on the graph path and
    86 groups over 8 waves (ragged) with streamed slots on the persistent path;
    the decode step is the 3B-width step run 16 times.  With the persistent
    step on 64 CUs, every GEMV CU holds more slots than it loads ahead (up to
    ~170 per wave), so most of its weights stream in during the phase, as at
    the 16K-context shape.  With the rank-16 adapter of the LoRA workload
    (alpha 32) the persistent step adds its LoRA-down CU.  8-token prompt,
    every step's logits checked."""
    from gpu_util import lora_to_device
    shape = QWEN25_INT4_2L
    log(f"3B-width int4, path={path}")
    w = synth.make_weights(shape, seed=45, random_gains=True)
    lora = synth.make_lora(shape, 16, seed=47) if path.endswith("lora") else None
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=32.0)
    if path == "persistent-64cu":
        monkeypatch.setenv("QD_PERSIST_CUS", "64")
    dec = make_decoder(torch_cuda, shape, 16, path.split("-")[0], lora_rank_max=16 if lora else 0)
    monkeypatch.delenv("QD_PERSIST_CUS", raising=False)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    del dw
    if lora:
        dec.set_lora(lora_to_device(lora), 16, 32.0)
    prompt = synth.make_prompt(shape.vocab, 8, seed=46)
    recs = lockstep_greedy(dec, oracle, prompt, 16, log=log)
    assert_records(recs, max_forced=1)
    dec.close()


# 16 kv heads of 8 q heads each: the decode attention cuts each kv head's
# positions into 256 / 16 = 16 splits, so near 2100 positions a split holds
# 132 positions, two full 64-position tiles and a ragged one
G8_WIDE = dataclasses.replace(synth.TINY, name="tiny-128q-16kv", n_q_heads=128, n_kv_heads=16, max_pos=2304)


@pytest.mark.parametrize("kv,rank", [("f32", 0), ("bf16", 12)])
def test_graph_attention_g8_several_tiles_per_split(torch_cuda, kv, rank):
    """Tiny model with 8 q heads per kv head and 16 kv heads on the graph path:
    past 2048 positions every split of the decode attention spans three
    64-position tiles (the last one ragged), so the kernel's tile loop, its
    next-tile requests and the new row's patch in a later tile all run.  With
    the bf16 cache and a rank-12 adapter (rank not a multiple of 8: B rows are
    not 16-byte aligned).  2100-token prompt (one batched prefill), then 10
    decode steps, every logit checked."""
    import decoder_only_token_amd as qd
    from gpu_util import lora_to_device
    shape = G8_WIDE
    log(f"graph G=8 attention, several tiles per split, kv={kv}, rank={rank}")
    w = synth.make_weights(shape, seed=48, random_gains=True)
    lora = synth.make_lora(shape, rank, seed=49) if rank else None
    oracle = OracleModel(shape, w, lora=lora, lora_alpha=24.0, kv_bf16=kv == "bf16")
    cfg = qd.make_config(shape, max_prefill=2112, lora_rank_max=rank, decode_path=PATHS["graph"],
                         kv_format=qd.QD_KV_BF16 if kv == "bf16" else qd.QD_KV_F32)
    dec = qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    del dw
    if lora:
        dec.set_lora(lora_to_device(lora), rank, 24.0)
    prompt = synth.make_prompt(shape.vocab, 2100, seed=50)
    recs = lockstep_greedy(dec, oracle, prompt, 10, log=log)
    assert_records(recs, max_forced=1)
    dec.close()


@pytest.mark.parametrize("nq", [32, 64])
def test_graph_prefill_eight_wave_attention(torch_cuda, nq):
    """16 kv heads with 2 or 4 q heads each: a 2100-row batched prefill gives
    at least two 128-query blocks per CU, so the batch attention runs its
    8-wave form (the last query tile ragged: 2100 = 32 x 65 + 20 rows at
    G = 2, 16 x 131 + 4 at G = 4); then 4 graph decode steps, every logit
    checked against the oracle."""
    import decoder_only_token_amd as qd
    shape = dataclasses.replace(synth.TINY, name=f"tiny-{nq}q-16kv", n_q_heads=nq, n_kv_heads=16, max_pos=2112)
    log(f"8-wave batch attention, nq={nq}, nkv=16, 2100-row prefill")
    w = synth.make_weights(shape, seed=51, random_gains=True)
    oracle = OracleModel(shape, w)
    cfg = qd.make_config(shape, max_prefill=2112, decode_path=PATHS["graph"])
    dec = qd.Decoder(cfg, torch_cuda.cuda.current_stream().cuda_stream)
    dw = to_device(w)
    torch_cuda.cuda.synchronize()
    dec.load_weights(dw)
    del dw
    prompt = synth.make_prompt(shape.vocab, 2100, seed=52)
    recs = lockstep_greedy(dec, oracle, prompt, 4, log=log)
    assert_records(recs, max_forced=1)
    dec.close()
