"""Pins of the CPU oracle to closed forms, hand-worked examples and invariants.

Every function of the oracle is checked here against something other than
itself, so that a dropped term, a wrong sign or index, or a transposed operand
fails at least one test.  Hand-worked values live in tests/golden/ with their
derivation.  No GPU is needed.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import (OracleModel, rmsnorm, rope_rotate, causal_gqa_attention, silu, swiglu_mlp,
                    argmax_lowest, quantize_int4_g128, dequantize_int4_g128, splitmix64_output,
                    quantize_q8_0, dequantize_q8_0,
                    uniform_for_step, sample_top_k_top_p)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def tiny_shape(**kw):
    base = dict(name="pin", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
                intermediate=96, vocab=80, max_pos=32)
    base.update(kw)
    return synth.ModelShape(**base)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_worked_example():
    g = golden("rmsnorm_worked.json")
    x = np.array(g["x"], dtype=np.float64)
    np.testing.assert_allclose(rmsnorm(x, np.ones(2), 0.0), g["want_unit_gain"], rtol=1e-14)
    np.testing.assert_allclose(rmsnorm(x, np.array(g["gain"]), 0.0), g["want_gain"], rtol=1e-14)


def test_rmsnorm_output_rms_closed_form():
    rng = np.random.default_rng(5)
    for m in (4, 128, 1024):
        x = rng.standard_normal((3, m)) * rng.uniform(0.01, 10, (3, 1))
        eps = 1e-6
        y = rmsnorm(x, np.ones(m), eps)
        ms = np.mean(x * x, axis=1)
        want = np.sqrt(ms / (ms + eps))
        np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), want, rtol=1e-13)


def test_rmsnorm_is_per_row_and_per_head():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 3, 8))
    x[:, 1] *= 100.0
    y = rmsnorm(x, np.ones(8), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), np.ones((2, 3)), rtol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_rope_worked_examples():
    g = golden("rope_worked.json")
    for c in g["cases"]:
        x = np.array(c["x"], dtype=np.float64).reshape(1, 1, g["d"])
        y = rope_rotate(x, np.array([c["pos"]]), g["theta"])
        np.testing.assert_allclose(y.reshape(-1), c["want"], rtol=0, atol=1e-15)


def test_rope_position_zero_is_identity_bit_exact():
    x = np.random.default_rng(1).standard_normal((1, 3, 128))
    assert np.array_equal(rope_rotate(x, np.array([0]), 1e6), x)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 2, 128))
    pos = np.array([1, 7, 100, 2047, 16383])
    y = rope_rotate(x, pos, 1e6)
    nx = x[..., :64] ** 2 + x[..., 64:] ** 2
    ny = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-12)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    for m, n, shift in ((5, 2, 11), (100, 0, 900), (3000, 2999, 13000)):
        a = np.sum(rope_rotate(q, np.array([m]), 1e6) * rope_rotate(k, np.array([n]), 1e6))
        b = np.sum(rope_rotate(q, np.array([m + shift]), 1e6) * rope_rotate(k, np.array([n + shift]), 1e6))
        assert abs(a - b) <= 1e-9 * (1 + abs(a))


# ---------------------------------------------------------------- attention

def test_attention_two_position_worked_example():
    g = golden("attention_two_position.json")
    d = g["d"]
    q = np.array([g["q"], g["q"]], dtype=np.float64).reshape(2, 1, d)
    k = np.array(g["k"], dtype=np.float64).reshape(2, 1, d)
    v = np.array(g["v"], dtype=np.float64).reshape(2, 1, d)
    o = causal_gqa_attention(q, k, v, np.array([0, 1]))
    np.testing.assert_allclose(o[0, 0], g["want_pos0"], rtol=1e-14)
    np.testing.assert_allclose(o[1, 0], g["want_pos1"], rtol=1e-14)


def test_attention_single_position_returns_v_exactly():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 2, 16))
    o = causal_gqa_attention(q, k, v, np.array([0]))
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[0, 3], v[0, 1])


def test_attention_gqa_head_mapping_consecutive():
    # kv head 0 carries value 1, kv head 1 carries value 2; q heads 0,1 -> kv 0; 2,3 -> kv 1
    rng = np.random.default_rng(7)
    T, d = 5, 8
    q = rng.standard_normal((T, 4, d))
    k = rng.standard_normal((T, 2, d))
    v = np.zeros((T, 2, d))
    v[:, 0] = 1.0
    v[:, 1] = 2.0
    o = causal_gqa_attention(q, k, v, np.arange(T))
    np.testing.assert_allclose(o[:, :2], 1.0, rtol=1e-14)
    np.testing.assert_allclose(o[:, 2:], 2.0, rtol=1e-14)


def test_attention_equal_scores_average_visible_values():
    T, d = 6, 8
    q = np.zeros((T, 2, d))
    k = np.random.default_rng(8).standard_normal((T, 1, d))
    v = np.arange(T, dtype=np.float64)[:, None, None] * np.ones((T, 1, d))
    o = causal_gqa_attention(q, k, v, np.arange(T))
    for p in range(T):
        np.testing.assert_allclose(o[p, :, 0], np.mean(np.arange(p + 1)), rtol=1e-14)


def test_attention_is_causal():
    rng = np.random.default_rng(9)
    T, d = 7, 16
    q = rng.standard_normal((T, 4, d))
    k = rng.standard_normal((T, 2, d))
    v = rng.standard_normal((T, 2, d))
    o1 = causal_gqa_attention(q, k, v, np.arange(T))
    k2, v2 = k.copy(), v.copy()
    k2[4:] += 3.0
    v2[4:] -= 5.0
    o2 = causal_gqa_attention(q, k2, v2, np.arange(T))
    assert np.array_equal(o1[:4], o2[:4])
    assert not np.allclose(o1[4:], o2[4:])


def test_attention_softmax_shift_invariance_and_brute_force():
    # brute force with an explicit TxT masked score matrix in pure Python, tiny sizes
    rng = np.random.default_rng(10)
    T, nq, nkv, d = 4, 2, 1, 3
    q = rng.standard_normal((T, nq, d))
    k = rng.standard_normal((T, nkv, d))
    v = rng.standard_normal((T, nkv, d))
    o = causal_gqa_attention(q, k, v, np.arange(T))
    for h in range(nq):
        for i in range(T):
            scores = [sum(q[i, h, c] * k[j, 0, c] for c in range(d)) / math.sqrt(d) if j <= i else -math.inf
                      for j in range(T)]
            w = [math.exp(s) for s in scores]
            tot = sum(w)
            want = [sum(w[j] * v[j, 0, c] for j in range(T)) / tot for c in range(d)]
            np.testing.assert_allclose(o[i, h], want, rtol=1e-12)


# ---------------------------------------------------------------- SiLU / MLP

def test_silu_and_mlp_worked_examples():
    g = golden("silu_worked.json")
    for z, want in g["silu"]:
        assert silu(np.array(float(z))) == pytest.approx(want, rel=1e-15, abs=0)
    got = swiglu_mlp(np.array([[1.0]]), np.array([[1.0]]), np.array([[2.0]]), np.array([[1.0]]))
    assert got[0, 0] == pytest.approx(g["mlp_gate1_up2_down1_h1"], rel=1e-15)
    assert got[0, 0] != pytest.approx(g["mlp_swapped"], rel=1e-6)


def test_silu_limits():
    assert silu(np.array(60.0)) == pytest.approx(60.0, rel=1e-15)
    assert abs(silu(np.array(-800.0))) < 1e-300


# ---------------------------------------------------------------- whole model

def _model(shape, weights, **kw):
    return OracleModel(shape, weights, **kw)


def test_zero_layer_model_is_tied_head_of_normalised_embedding():
    # Hadamard rows: orthogonal, all of norm 2 -> logits[t] = 4/sqrt(1+eps), others 0
    shape = tiny_shape(n_layers=0, hidden=4, vocab=4, n_q_heads=1, n_kv_heads=1, head_dim=4, intermediate=4)
    had = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float32)
    w = {"embed": synth.bf16_round(had), "final_norm": synth.bf16_round(np.ones(4, np.float32)), "layers": []}
    m = _model(shape, w)
    logits = m.forward([2])
    want = np.zeros(4)
    want[2] = 4.0 / math.sqrt(1.0 + shape.rms_eps)
    np.testing.assert_allclose(logits[0], want, rtol=1e-15, atol=1e-15)
    assert argmax_lowest(logits[0]) == 2


def test_zero_layer_model_applies_final_norm_gains():
    shape = tiny_shape(n_layers=0, hidden=4, vocab=4, n_q_heads=1, n_kv_heads=1, head_dim=4, intermediate=4)
    had = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=np.float32)
    gains = np.array([0.5, 2.0, 1.5, 3.0], dtype=np.float32)
    w = {"embed": synth.bf16_round(had), "final_norm": synth.bf16_round(gains), "layers": []}
    logits = _model(shape, w).forward([1])[0]
    want = np.array([sum(float(had[v, j]) * float(gains[j]) * float(had[1, j]) for j in range(4))
                     for v in range(4)]) / math.sqrt(1.0 + shape.rms_eps)
    np.testing.assert_allclose(logits, want, rtol=1e-15, atol=1e-15)


def test_mlp_wiring_single_position():
    # With o_proj zero, a layer is x + down(SiLU(gate h2) * up h2), h2 = RMSNorm(x; mlp gains).
    shape = tiny_shape(n_layers=1)
    w = synth.make_weights(shape, seed=29, random_gains=True)
    w["layers"][0]["wo"] = np.zeros_like(w["layers"][0]["wo"])
    cap = {}
    _model(shape, w).forward([3], capture=cap)
    f = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    lw = w["layers"][0]
    x = f(w["embed"])[3]
    h2 = x / np.sqrt(np.mean(x * x) + shape.rms_eps) * f(lw["mlp_norm"])
    g = f(lw["w_gate"]) @ h2
    u = f(lw["w_up"]) @ h2
    want = x + f(lw["w_down"]) @ (g / (1.0 + np.exp(-g)) * u)
    np.testing.assert_allclose(cap["layer_out"][0][0], want, rtol=1e-12, atol=1e-14)


def test_zero_projection_layers_are_identity_on_the_bus():
    shape = tiny_shape()
    w = synth.make_weights(shape, seed=11)
    base = _model(dataclasses.replace(shape, n_layers=0), {"embed": w["embed"], "final_norm": w["final_norm"],
                                                             "layers": []})
    for lw in w["layers"]:
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            lw[name] = np.zeros_like(lw[name])
    full = _model(shape, w)
    toks = synth.make_prompt(shape.vocab, 6, seed=12)
    np.testing.assert_allclose(full.forward(toks), base.forward(toks), rtol=1e-14, atol=1e-14)


def test_single_position_layer_closed_form():
    # At position 0 attention returns v exactly, so one layer with zero MLP is
    # x + Wo (Wv rmsnorm(x) + bv): pins V (not K or Q), bias, o_proj orientation, residual base.
    shape = tiny_shape(n_layers=1, qkv_bias=True, qk_norm=False)
    w = synth.make_weights(shape, seed=13, random_gains=True)
    for name in ("w_gate", "w_up", "w_down"):
        w["layers"][0][name] = np.zeros_like(w["layers"][0][name])
    m = _model(shape, w)
    cap = {}
    m.forward([7], capture=cap)
    f = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    lw = w["layers"][0]
    x = f(w["embed"])[7]
    h = x / np.sqrt(np.mean(x * x) + shape.rms_eps) * f(lw["attn_norm"])
    v = f(lw["wv"]) @ h + f(lw["bv"])
    vrep = np.repeat(v.reshape(shape.n_kv_heads, shape.head_dim), shape.n_q_heads // shape.n_kv_heads, axis=0)
    want = x + f(lw["wo"]) @ vrep.reshape(-1)
    np.testing.assert_allclose(cap["layer_out"][0][0], want, rtol=1e-12, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv_heads():
    shape = tiny_shape(n_q_heads=4, n_kv_heads=2)
    w = synth.make_weights(shape, seed=14, random_gains=True)
    mha_shape = dataclasses.replace(shape, n_kv_heads=4)
    w2 = {"embed": w["embed"], "final_norm": w["final_norm"], "layers": []}
    d = shape.head_dim
    for lw in w["layers"]:
        l2 = dict(lw)
        for name in ("wk", "wv"):
            heads = lw[name].reshape(2, d, shape.hidden)
            l2[name] = np.repeat(heads, 2, axis=0).reshape(4 * d, shape.hidden)
        w2["layers"].append(l2)
    toks = synth.make_prompt(shape.vocab, 9, seed=15)
    np.testing.assert_allclose(_model(shape, w).forward(toks), _model(mha_shape, w2).forward(toks),
                               rtol=1e-12, atol=1e-13)


def test_qk_norm_makes_logits_invariant_to_scaling_q_and_k_weights():
    shape = tiny_shape()
    w = synth.make_weights(shape, seed=16)
    toks = synth.make_prompt(shape.vocab, 8, seed=17)
    ref = _model(shape, w).forward(toks)
    for lw in w["layers"]:
        for name in ("wq", "wk"):
            lw[name] = synth.bf16_round(synth.bf16_to_f32(lw[name]) * np.float32(4.0))  # exact power-of-two scale
    got = _model(shape, w).forward(toks)
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-5)
    no_norm = dataclasses.replace(shape, qk_norm=False)
    w2 = synth.make_weights(no_norm, seed=16)
    a = _model(no_norm, w2).forward(toks)
    for lw in w2["layers"]:
        for name in ("wq", "wk"):
            lw[name] = synth.bf16_round(synth.bf16_to_f32(lw[name]) * np.float32(4.0))
    b = _model(no_norm, w2).forward(toks)
    assert np.max(np.abs(a - b)) > 1e-4


def _qk_layer_by_hand(w, shape, toks, order="norm_then_rope", swap=False):
    """One layer with a zero MLP at two positions, written out from the block
    figure of "Failed Star / fs — Forward pass → logits" (QK-norm, then RoPE,
    then causal GQA attention) with RoPE as a complex rotation of
    a_j + i b_j (half-split pairs) and a two-entry softmax; returns the layer
    output of position 1.  `order` / `swap` build deliberately wrong variants."""
    f = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    lw = w["layers"][0]
    d, nq, nkv, eps = shape.head_dim, shape.n_q_heads, shape.n_kv_heads, shape.rms_eps
    gq, gk = f(lw["q_norm"]), f(lw["k_norm"])
    if swap:
        gq, gk = gk, gq
    xs = [f(w["embed"])[t] for t in toks]
    qs, ks, vs = [], [], []
    for p, x in enumerate(xs):
        h = f(lw["attn_norm"]) * x / math.sqrt(float(np.dot(x, x)) / x.size + eps)
        q = (f(lw["wq"]) @ h).reshape(nq, d)
        k = (f(lw["wk"]) @ h).reshape(nkv, d)
        vs.append((f(lw["wv"]) @ h).reshape(nkv, d))

        def rot(u):
            z = u[:d // 2] + 1j * u[d // 2:]
            z = z * np.exp(1j * p * (shape.rope_theta ** (-2.0 * np.arange(d // 2) / d)))
            return np.concatenate([z.real, z.imag])

        def nrm(u, g):
            return g * u / math.sqrt(float(np.dot(u, u)) / d + eps)

        if order == "norm_then_rope":
            qs.append(np.stack([rot(nrm(q[i], gq)) for i in range(nq)]))
            ks.append(np.stack([rot(nrm(k[i], gk)) for i in range(nkv)]))
        else:
            qs.append(np.stack([nrm(rot(q[i]), gq) for i in range(nq)]))
            ks.append(np.stack([nrm(rot(k[i]), gk) for i in range(nkv)]))
    o = np.zeros((nq, d))
    for hh in range(nq):
        g = hh // (nq // nkv)
        s0 = float(np.dot(qs[1][hh], ks[0][g])) / math.sqrt(d)
        s1 = float(np.dot(qs[1][hh], ks[1][g])) / math.sqrt(d)
        p1 = 1.0 / (1.0 + math.exp(s0 - s1))
        o[hh] = (1.0 - p1) * vs[0][g] + p1 * vs[1][g]
    return xs[1] + f(lw["wo"]) @ o.reshape(-1)


def test_qk_norm_gains_and_order_closed_form():
    # Distinct random q_norm / k_norm gains; the hand-written layer (complex
    # RoPE, explicit two-entry softmax) must equal the oracle, and swapping the
    # gains or rotating before normalising must not.
    shape = tiny_shape(n_layers=1, qk_norm=True)
    w = synth.make_weights(shape, seed=31, random_gains=True)
    lw = w["layers"][0]
    rng = np.random.default_rng(32)
    lw["q_norm"] = synth.bf16_round(rng.uniform(0.3, 2.5, shape.head_dim).astype(np.float32))
    lw["k_norm"] = synth.bf16_round(rng.uniform(0.3, 2.5, shape.head_dim).astype(np.float32))
    for name in ("w_gate", "w_up", "w_down"):
        lw[name] = np.zeros_like(lw[name])
    toks = [11, 42]
    cap = {}
    _model(shape, w).forward(toks, capture=cap)
    got = cap["layer_out"][0][1]
    want = _qk_layer_by_hand(w, shape, toks)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    for variant in (dict(swap=True), dict(order="rope_then_norm")):
        wrong = _qk_layer_by_hand(w, shape, toks, **variant)
        assert np.max(np.abs(wrong - got)) > 1e-6, variant


def test_incremental_equals_cacheless_prefill():
    shape = tiny_shape(qkv_bias=True)
    w = synth.make_weights(shape, seed=18, random_gains=True)
    m = _model(shape, w)
    toks = synth.make_prompt(shape.vocab, 12, seed=19)
    full = m.forward(toks)
    cache = m.new_cache()
    rows = [m.forward(toks[:5], cache)]
    for t in toks[5:]:
        rows.append(m.forward([t], cache))
    inc = np.concatenate(rows, axis=0)
    np.testing.assert_allclose(inc, full, rtol=1e-12, atol=1e-13)


def test_model_is_causal():
    shape = tiny_shape()
    m = _model(shape, synth.make_weights(shape, seed=20))
    toks = synth.make_prompt(shape.vocab, 10, seed=21)
    a = m.forward(toks)
    toks2 = toks.copy()
    toks2[6:] = (toks2[6:] + 1) % shape.vocab
    b = m.forward(toks2)
    np.testing.assert_allclose(a[:6], b[:6], rtol=1e-13, atol=1e-14)
    assert not np.allclose(a[6:], b[6:])


def test_lora_equals_merged_weights_and_zero_b_is_base():
    shape = tiny_shape(qk_norm=False, qkv_bias=True)
    w = synth.make_weights(shape, seed=22)
    lora = synth.make_lora(shape, rank=4, seed=23)
    toks = synth.make_prompt(shape.vocab, 7, seed=24)
    alpha = 8.0
    with_lora = _model(shape, w, lora=lora, lora_alpha=alpha).forward(toks)
    # merged: W' = W + (alpha/r) B A, computed in float64 by patching the oracle's widened weights
    merged = _model(shape, w)
    for li, lw in enumerate(lora):
        f = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa
        merged.layers[li]["wq"] = merged.layers[li]["wq"] + (alpha / 4) * f(lw["b_q"]) @ f(lw["a_q"])
        merged.layers[li]["wv"] = merged.layers[li]["wv"] + (alpha / 4) * f(lw["b_v"]) @ f(lw["a_v"])
    np.testing.assert_allclose(with_lora, merged.forward(toks), rtol=1e-11, atol=1e-12)
    zero_b = [dict(lw, b_q=np.zeros_like(lw["b_q"]), b_v=np.zeros_like(lw["b_v"])) for lw in lora]
    base = _model(shape, w).forward(toks)
    assert np.array_equal(_model(shape, w, lora=zero_b, lora_alpha=alpha).forward(toks), base)
    assert not np.allclose(with_lora, base)


def test_int4_model_uses_dequantised_projections():
    shape = tiny_shape(qk_norm=False, qkv_bias=True, hidden=128, intermediate=256, head_dim=32,
                       weight_format=synth.W_INT4_G128)
    w = synth.make_weights(shape, seed=25)
    m = _model(shape, w)
    f32 = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    codes, scales = quantize_int4_g128(f32(w["layers"][1]["w_down"]))
    np.testing.assert_array_equal(m.layers[1]["w_down"], codes.astype(np.float64) *
                                  np.repeat(scales.astype(np.float64), 128, axis=1))
    # biases, norms and the embedding stay bf16
    np.testing.assert_array_equal(m.layers[0]["bq"], f32(w["layers"][0]["bq"]).astype(np.float64))


# ---------------------------------------------------------------- greedy / sampling

def test_argmax_ties_go_to_lowest_index():
    assert argmax_lowest(np.array([1.0, 3.0, 2.0, 3.0])) == 1
    assert argmax_lowest(np.array([-1.0, -1.0])) == 0


def test_splitmix64_published_vectors():
    g = golden("splitmix64_vectors.json")
    got = [splitmix64_output(g["seed"], i + 1) for i in range(len(g["outputs_hex"]))]
    assert got == [int(h, 16) for h in g["outputs_hex"]]
    u = [uniform_for_step(2, s) for s in range(1000)]
    assert min(u) >= 0.0 and max(u) < 1.0 and abs(np.mean(u) - 0.5) < 0.03


def test_uniform_for_step_published_vectors():
    # u for step s is output s+1's top 24 bits over 2^24, derived by hand from
    # the published outputs: pins the counter offset and the bit window.
    g = golden("uniform_vectors.json")
    for s, (top, u) in enumerate(zip(g["top24"], g["u"])):
        assert uniform_for_step(g["seed"], s) == u == top / float(1 << 24), s


def test_sampling_worked_examples():
    g = golden("sampling_worked.json")
    logits = np.array(g["logits"])
    for c in g["cases"]:
        assert sample_top_k_top_p(logits, c["T"], c["top_k"], c["top_p"], c["u"]) == c["want"], c


def test_sampling_reduces_to_greedy():
    rng = np.random.default_rng(26)
    logits = rng.standard_normal(1000)
    best = argmax_lowest(logits)
    for u in (0.0, 0.3, 0.999):
        assert sample_top_k_top_p(logits, 0.7, 1, 0.9, u) == best
        assert sample_top_k_top_p(logits, 1e-6, 40, 0.9, u) == best
        assert sample_top_k_top_p(logits, 0.7, 40, 1e-9, u) == best


def test_sampling_distribution_matches_truncated_softmax():
    rng = np.random.default_rng(27)
    logits = rng.standard_normal(200) * 2.0
    T, k, p = 0.7, 40, 0.9
    n = 200000
    counts = {}
    for i in range(n):
        t = sample_top_k_top_p(logits, T, k, p, (i + 0.5) / n)
        counts[t] = counts.get(t, 0) + 1
    order = sorted(range(200), key=lambda i: (-logits[i], i))[:k]
    w = np.array([math.exp((logits[i] - logits[order[0]]) / T) for i in order])
    pi = w / w.sum()
    kept, before = [], 0.0
    for i, pr in zip(order, pi):
        if before < p or not kept:
            kept.append((i, pr))
        before += pr
    z = sum(pr for _, pr in kept)
    assert set(counts) == {i for i, _ in kept}
    for i, pr in kept:
        assert abs(counts[i] / n - pr / z) < 2.0 / n + 1e-12


# ---------------------------------------------------------------- int4 group-128

def test_int4_worked_example():
    g = golden("int4_worked.json")
    w = np.zeros((2, 128), dtype=np.float32)
    w[0, :len(g["values"])] = np.array(g["values"], dtype=np.float32)
    codes, scales = quantize_int4_g128(w)
    assert float(scales[0, 0]) == g["scale"]
    assert list(codes[0, :len(g["codes"])]) == g["codes"]
    assert np.all(codes[0, len(g["codes"]):] == 0)
    assert float(scales[1, 0]) == 0.0 and np.all(codes[1] == 0)


def test_int4_properties():
    rng = np.random.default_rng(28)
    w = synth.bf16_to_f32(synth.bf16_round(rng.standard_normal((64, 512)).astype(np.float32) * 0.02))
    codes, scales = quantize_int4_g128(w)
    assert codes.min() >= -7 and codes.max() <= 7
    s = np.repeat(scales.astype(np.float32), 128, axis=1)
    what = dequantize_int4_g128(codes, scales)
    # error within half a step (plus the float32 rounding of the division)
    assert np.all(np.abs(w - what) <= s * (0.5 + 1e-3))
    # the largest magnitude in each group maps to +-7
    g = np.abs(codes.reshape(64, 4, 128)).max(axis=2)
    assert np.all(g == 7)
    # idempotent: quantising the dequantised weights returns the same codes and scales
    c2, s2 = quantize_int4_g128(what.astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


# ---------------------------------------------------------------- Q8_0 (int8 blocks of 32)

def test_q8_0_worked_example():
    g = golden("q8_0_worked.json")
    w = np.zeros((2, 64), dtype=np.float32)
    w[0, :len(g["values"])] = np.array(g["values"], dtype=np.float32)
    w[0, 32:] = np.float32(0.5)  # a second block of the row: its own scale
    codes, scales = quantize_q8_0(w)
    assert float(scales[0, 0]) == g["scale"]
    assert scales[0, 0].view(np.uint16) == 0x211F
    assert list(codes[0, :len(g["codes"])]) == g["codes"]
    assert np.all(codes[0, len(g["codes"]):32] == 0)
    assert np.all(codes[0, 32:] == 127)  # the block's largest magnitude -> 127
    assert float(scales[1, 0]) == 0.0 and np.all(codes[1] == 0)


def test_q8_0_properties():
    rng = np.random.default_rng(29)
    w = synth.bf16_to_f32(synth.bf16_round(rng.standard_normal((48, 256)).astype(np.float32) * 0.02))
    w[3, 64:96] = 0.0  # an all-zero block
    codes, scales = quantize_q8_0(w)
    assert codes.dtype == np.int8 and codes.min() >= -127 and codes.max() <= 127
    assert scales.shape == (48, 8)
    s = np.repeat(scales.astype(np.float32), 32, axis=1)
    what = dequantize_q8_0(codes, scales)
    # error within half a step (plus the float32 rounding of the division)
    assert np.all(np.abs(w - what) <= s * (0.5 + 1e-3))
    # the largest magnitude of every non-zero block maps to +-127
    blk = np.abs(codes.reshape(48, 8, 32)).max(axis=2)
    nz = scales.astype(np.float32) > 0
    assert np.all(blk[nz] == 127) and np.all(blk[~nz] == 0) and not nz[3, 2]
    # idempotent: quantising the dequantised weights returns the same codes and scales
    c2, s2 = quantize_q8_0(what.astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # blocks are independent: changing one block leaves the others' codes alone
    w2 = w.copy()
    w2[5, 0:32] *= 3.0
    c3, s3 = quantize_q8_0(w2)
    assert np.array_equal(c3[:, 32:], codes[:, 32:]) and np.array_equal(c3[:5], codes[:5])


def test_q8_0_model_uses_dequantised_projections():
    shape = tiny_shape(qk_norm=True, qkv_bias=False, hidden=128, intermediate=256, head_dim=32,
                       weight_format=synth.W_Q8_0)
    w = synth.make_weights(shape, seed=26)
    m = _model(shape, w)
    f32 = lambda b: (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    for name in ("wq", "wo", "w_down"):
        codes, scales = quantize_q8_0(f32(w["layers"][0][name]))
        np.testing.assert_array_equal(m.layers[0][name], codes.astype(np.float64) *
                                      np.repeat(scales.astype(np.float64), 32, axis=1))
    # norms and the embedding stay bf16
    np.testing.assert_array_equal(m.layers[0]["attn_norm"], f32(w["layers"][0]["attn_norm"]).astype(np.float64))


@pytest.mark.parametrize("shape_name,lora", [("TINY", False), ("TINY_INT4", True)])
def test_layer_rows_matches_the_full_forward(shape_name, lora):
    """The row-sampled single-layer oracle used for full-size GPU checks gives,
    for the selected rows, exactly the layer outputs of the whole forward
    (same inputs, same definition restricted to those rows)."""
    import dataclasses
    shape = dataclasses.replace(getattr(synth, shape_name), n_layers=2)
    w = synth.make_weights(shape, seed=81, random_gains=True)
    lo = synth.make_lora(shape, 4, seed=82) if lora else None
    m = OracleModel(shape, w, lora=lo, lora_alpha=8.0 if lora else 0.0)
    prompt = synth.make_prompt(shape.vocab, 23, seed=83)
    cap = {}
    m.forward(prompt, capture=cap)
    rows = [0, 5, 22, 11]
    for li in range(shape.n_layers):
        x_in = cap["embed"] if li == 0 else cap["layer_out"][li - 1]
        got = m.layer_rows(li, x_in, rows)
        np.testing.assert_allclose(got, cap["layer_out"][li][rows], rtol=1e-12, atol=1e-12)


def test_round_bf16_hand_values():
    """bf16 keeps 8 significant bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7
    and goes to the even one (1); 1 + 3 2^-9 rounds up to 1 + 2^-7; signs and
    powers of two pass through; the step doubles with each binade (2^-6 in
    [2, 4), 8 in [1024, 2048))."""
    from oracle import round_bf16
    cases = {1.0: 1.0, 1.0 + 2 ** -8: 1.0, 1.0 + 3 * 2 ** -9: 1.0 + 2 ** -7, 1.0 + 2 ** -7: 1.0 + 2 ** -7,
             1.0 + 3 * 2 ** -8: 1.0 + 2 ** -6, -1.0 - 2 ** -8: -1.0, 2.0 + 2 ** -7: 2.0,
             3.0 + 2 ** -7: 3.0,  # half a step (2^-6 in [2, 4)) above 3, whose last bit is even
             3.0 + 3 * 2 ** -8: 3.0 + 2 ** -6, 1024.0 + 3.0: 1024.0, 1024.0 + 5.0: 1032.0,  # steps of 8
             0.0: 0.0, -0.5: -0.5, 2 ** -100: 2 ** -100}
    for x, want in cases.items():
        assert round_bf16(np.array([x]))[0] == want, x


def test_round_bf16_matches_the_float32_bit_rule():
    """On float32 inputs, round_bf16 equals rounding the float32 bit pattern to
    its top 16 bits (round half to even on the dropped 16 bits) — an integer
    rule independent of the frexp form used by the oracle."""
    from oracle import round_bf16
    rng = np.random.default_rng(40)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    x[:4] = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 65504.0], dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    want = r.astype(np.uint32).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(round_bf16(x.astype(np.float64)), want)


def test_kv_bf16_model_reads_back_rounded_keys_and_values():
    """With a bf16 cache the decode step's output equals the f32-cache model's
    exactly when every cached key and value is already a bf16 value (here:
    zero q/k/v weights and k bias, so k = 0 and v is its bf16 bias);
    and a decode from a cache filled at prefill equals the cache-less forward
    (the rounding happens once, at the store)."""
    shape = tiny_shape(qkv_bias=True)
    w = synth.make_weights(shape, seed=41, random_gains=True)
    toks = synth.make_prompt(shape.vocab, 9, seed=42)
    m = OracleModel(shape, w, kv_bf16=True)
    full = m.forward(toks)
    cache = m.new_cache()
    inc = np.concatenate([m.forward(toks[:4], cache)] + [m.forward([t], cache) for t in toks[4:]], axis=0)
    np.testing.assert_allclose(inc, full, rtol=1e-12, atol=1e-13)
    # the rounding is actually applied, and it is small
    f32 = OracleModel(shape, w).forward(toks)
    d = np.max(np.abs(f32 - full))
    assert 0 < d < 0.05 * np.max(np.abs(f32))
    # keys and values that are bf16 already: identical to the f32 cache
    w2 = synth.make_weights(shape, seed=43)
    for lw in w2["layers"]:  # k = 0 and v = its bf16 bias on every row
        for nm in ("wq", "wk", "wv", "bk"):
            lw[nm] = np.zeros_like(lw[nm])
    a = OracleModel(shape, w2, kv_bf16=True).forward(toks)
    b = OracleModel(shape, w2).forward(toks)
    np.testing.assert_array_equal(a, b)
