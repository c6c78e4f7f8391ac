"""C-ABI checks that need no GPU: the library loads, exports every function
include/qd.h declares, the ctypes mirrors match the C struct sizes, and
qd_create rejects bad configurations before making any HIP call."""
import ctypes
import dataclasses
import os
import re

import pytest

import synth
import decoder_only_token_amd as qd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(qd_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_function():
    lib = qd.load_library()
    names = declared_functions()
    assert {"qd_create", "qd_load_weights", "qd_prefill", "qd_decode_step", "qd_reset_kv"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(qd.EXPORTS) == names


def test_struct_sizes_match_ctypes_mirrors():
    lib = qd.load_library()
    assert lib.qd_sizeof_config() == ctypes.sizeof(qd.QdConfig)
    assert lib.qd_sizeof_weights() == ctypes.sizeof(qd.QdWeights)
    assert lib.qd_sizeof_sampling() == ctypes.sizeof(qd.QdSampling)
    assert lib.qd_sizeof_lora() == ctypes.sizeof(qd.QdLora)


def _create(cfg):
    lib = qd.load_library()
    h = ctypes.c_void_p()
    return lib.qd_create(ctypes.byref(cfg), None, ctypes.byref(h)), h


@pytest.mark.parametrize("mutate,code", [
    (lambda c: setattr(c, "struct_size", c.struct_size - 4), -2),
    (lambda c: setattr(c, "abi_version", 99), -2),
    (lambda c: setattr(c, "head_dim", 64), -1),
    (lambda c: setattr(c, "n_kv_heads", 3), -1),
    (lambda c: setattr(c, "n_layers", 0), -1),
    (lambda c: setattr(c, "max_prefill", 0), -1),
    (lambda c: setattr(c, "max_prefill", c.max_pos + 1), -1),
    (lambda c: setattr(c, "tie_embeddings", 0), -1),
    (lambda c: setattr(c, "rope_theta", 0.0), -1),
])
def test_create_rejects_bad_config_before_any_hip_call(mutate, code):
    cfg = qd.make_config(synth.TINY, max_prefill=16)
    mutate(cfg)
    rc, h = _create(cfg)
    assert rc == code
    assert not h.value


def test_unknown_weight_format_is_rejected():
    cfg = qd.make_config(synth.TINY_INT4, max_prefill=16)
    cfg.weight_format = 7
    rc, h = _create(cfg)
    assert rc == -1 and not h.value


def test_lora_rank_bounds_per_decode_path():
    """The persistent step's LoRA-down CU holds [A_q; A_v] in its 24 register
    slots per lane: ceil(r / 4) * hidden / 512 <= 24 (r <= 48 at hidden 1024,
    r <= 24 at 2048); the graph path takes r <= 64.  Rejected before any HIP call."""
    big = dataclasses.replace(synth.TINY, hidden=2048)
    for shape, r in ((synth.TINY, 49), (big, 25)):
        cfg = qd.make_config(shape, max_prefill=16, lora_rank_max=r, decode_path=qd.QD_DECODE_PERSISTENT)
        rc, h = _create(cfg)
        assert rc == -1 and not h.value, (shape.hidden, r)
    cfg = qd.make_config(synth.TINY, max_prefill=16, lora_rank_max=65, decode_path=qd.QD_DECODE_GRAPH)
    rc, h = _create(cfg)
    assert rc == -1 and not h.value
    err = qd.load_library().qd_last_error(None)
    assert isinstance(err, bytes)


def test_create_rejects_null_config():
    lib = qd.load_library()
    h = ctypes.c_void_p()
    assert lib.qd_create(None, None, ctypes.byref(h)) == -1


def test_null_handle_calls_fail_cleanly():
    lib = qd.load_library()
    assert lib.qd_reset_kv(None) == -1
    assert lib.qd_decode_step(None, None, None, None) == -1
    assert lib.qd_prefill(None, None, 0, None, None, None) == -1
    assert isinstance(lib.qd_last_error(None), bytes)  # the handle-free calls' last reason
    lib.qd_destroy(None)


def test_persistent_path_rejects_more_than_254_layers():
    # the persistent step's handshake tags hold the layer in 8 bits (255 is reserved)
    cfg = qd.make_config(synth.TINY, max_prefill=16, decode_path=qd.QD_DECODE_PERSISTENT)
    cfg.n_layers = 255
    rc, h = _create(cfg)
    assert rc == -1 and not h.value
    cfg.n_layers = 254
    rc, h = _create(cfg)
    assert rc != -1  # passes validation (no GPU here: fails later, at the first HIP call)
    if rc == 0:
        qd.load_library().qd_destroy(h)


def test_abandoned_count_needs_an_output_pointer():
    lib = qd.load_library()
    assert lib.qd_get_abandoned(None, None) == -1


def _sample_call(logits=1 << 20, vocab=1000, sampling=None, token=1 << 21, ws=1 << 22, ws_bytes=1 << 20):
    lib = qd.load_library()
    return lib.qd_sample_logits(logits, vocab, None if sampling is None else ctypes.byref(sampling), 0, token, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), -1),
    (dict(token=None), -1),
    (dict(ws=None), -1),
    (dict(vocab=0), -1),
    (dict(vocab=524289), -1),
    (dict(ws_bytes=7), -1),
    (dict(ws=(1 << 22) + 2), -1),
    (dict(sampling=qd.make_sampling(0.7, 0, 0.9, 1)), -1),
    (dict(sampling=qd.make_sampling(0.7, 65, 0.9, 1)), -1),
    (dict(sampling=qd.make_sampling(0.7, 40, 0.0, 1)), -1),
    (dict(sampling=qd.make_sampling(float("inf"), 40, 0.9, 1)), -1),
    (dict(vocab=16, sampling=qd.make_sampling(0.7, 40, 0.9, 1)), -1),
])
def test_handle_free_sampler_checks_arguments_before_any_hip_call(kw, code):
    """Every bad argument is refused (with a reason) before the library
    touches the device, so these run without a GPU."""
    assert _sample_call(**kw) == code
    assert qd.load_library().qd_last_error(None)


def test_handle_free_sampler_rejects_a_foreign_struct_size():
    s = qd.make_sampling(0.7, 40, 0.9, 1)
    s.struct_size -= 4
    assert _sample_call(sampling=s) == -2


def test_sampler_workspace_size():
    """K lists of (value, id) per 1024-logit slice: greedy keeps one entry."""
    assert qd.sample_workspace_bytes(151936) == 149 * 1 * 8
    assert qd.sample_workspace_bytes(151936, qd.make_sampling(0.7, 40, 0.9, 1)) == 149 * 40 * 8
    assert qd.sample_workspace_bytes(1025, qd.make_sampling(0.0, 0, 0.0, 1)) == 2 * 8
    assert qd.sample_workspace_bytes(0) == 0
    assert qd.sample_workspace_bytes(8, qd.make_sampling(0.7, 9, 0.9, 1)) == 0
    assert qd.sample_workspace_bytes(524288, qd.make_sampling(0.7, 39, 0.9, 1)) == 512 * 39 * 8
    assert qd.sample_workspace_bytes(524288, qd.make_sampling(0.7, 40, 0.9, 1)) == 0  # merge LDS bound


def test_q8_0_weights_need_the_graph_path():
    """QD_W_Q8_0 runs on the graph decode path only (refused on the persistent
    step before any HIP call); make_config picks the graph for it by default."""
    cfg = qd.make_config(synth.TINY_Q8, max_prefill=16, decode_path=qd.QD_DECODE_PERSISTENT)
    rc, h = _create(cfg)
    assert rc == -1 and not h.value
    assert qd.make_config(synth.TINY_Q8, max_prefill=16).decode_path == qd.QD_DECODE_GRAPH
    assert qd.make_config(synth.TINY, max_prefill=16).decode_path == qd.QD_DECODE_PERSISTENT
    cfg = qd.make_config(synth.TINY, max_prefill=16)
    cfg.weight_format = 3
    rc, h = _create(cfg)
    assert rc == -1 and not h.value


def test_bf16_kv_cache_needs_the_graph_path():
    """kv_format QD_KV_BF16 runs on the graph decode path only, and unknown
    formats are refused; both before any HIP call."""
    cfg = qd.make_config(synth.TINY, max_prefill=16, decode_path=qd.QD_DECODE_PERSISTENT, kv_format=qd.QD_KV_BF16)
    rc, h = _create(cfg)
    assert rc == -1 and not h.value
    cfg = qd.make_config(synth.TINY, max_prefill=16, decode_path=qd.QD_DECODE_GRAPH, kv_format=2)
    rc, h = _create(cfg)
    assert rc == -1 and not h.value


def test_greedy_acceptance_rule():
    """Leading drafts equal to the choice before them are accepted."""
    assert qd.accepted_drafts([5, 6, 7], [5, 6, 7, 8]) == 3
    assert qd.accepted_drafts([5, 6, 7], [5, 9, 7, 8]) == 1
    assert qd.accepted_drafts([5, 6, 7], [4, 6, 7, 8]) == 0
    assert qd.accepted_drafts([], [3]) == 0
