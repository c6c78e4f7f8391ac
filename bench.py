"""Benchmark: single-sequence decode (and prefill) of a Qwen-style decoder on one MI355X.

Headline workload (default): qwen2.5-3b-int4-lora, the largest one-GPU
configuration (36 layers, hidden 2048, 16/2 heads, int4 group-128 projection
weights, rank-16 LoRA on q/v, 16,384-position f32 KV cache).  One timed step
is one decode token at the end of the context: the cache is filled untimed
(the workload's 8192-token prompt as one batched prefill, then batched
prefills of random tokens) to 16384 - warmup - steps positions, then `warmup`
untimed and `steps` timed decode steps run back to back on one HIP stream
(device-resident token feedback, one host synchronisation at the end), the
last one reaching position 16383.  Weights, prompt and cache are resident in
HBM before timing starts.

Prints ONE JSON line: `value` = decode tokens / second over the timed steps;
beside it the roofline of the decode kernel (algorithmic bytes per step =
weights + LoRA factors + tied LM head + one embedding row + KV read and
write, over the step's measured time), the workload's batched prefill
(tokens / s, projection TFLOP/s, MFMA use), the qwen3-0.6b decode job of the
previous measurements as extra keys, and the CPU oracle timed on a bounded
sample of the same decode step (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_BF16_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen2.5-3b-int4-lora")
    ap.add_argument("--path", choices=["auto", "persistent", "graph"], default="auto",
                    help="decode step as one persistent kernel, or as per-operation kernels in a hipGraph "
                         "(auto: the persistent kernel without an adapter, the graph with one or with Q8_0 weights)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the qwen3-0.6b job and the prefill timing")
    ap.add_argument("--only-decode", action="store_true", help="decode timing only (for profiler runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 launches): the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# Sources of the persistent decode kernel: HBM traffic measured with counters
# is reported only while these are unchanged since the counters were taken.
KERNEL_SOURCES = ["decoder_only_token_amd/csrc/persist.hip", "decoder_only_token_amd/csrc/persist.h",
                  "decoder_only_token_amd/csrc/common.h"]


def kernel_source_hash(files=None) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def library_sources():
    """Every source of the HIP library (the graph path's kernels), sorted."""
    d = os.path.join(ROOT, "decoder_only_token_amd", "csrc")
    return sorted(os.path.join("decoder_only_token_amd", "csrc", f) for f in os.listdir(d)
                  if f.endswith((".hip", ".h")))


def measured_traffic(workload: str, path: str = "persistent"):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel factor): per launch of the
    persistent decode kernel, or per decode step (every kernel of the captured
    graph) on the graph path; None when there is none for this workload or the
    sources have changed since."""
    if path == "graph":
        fname, key, want = f"decode_graph.{workload}.traffic.txt", "library_source_sha256_16", \
            kernel_source_hash(library_sources())
    else:
        fname, key, want = f"k_decode_persistent.{workload}.traffic.txt", "kernel_source_sha256_16", \
            kernel_source_hash()
    fpath = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(fpath):
        return None
    kv = {}
    with open(fpath) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get(key) != want:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibrate_copy(mib: int):
    import torch
    n = mib * 1024 * 1024 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n * 4,
                      "bytes_written_per_launch": n * 4, "launches": 5}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def step_bytes(shape, lora_rank, ctx, kv_elem_bytes=4):
    """Algorithmic HBM bytes of one decode step whose context after the step is
    ctx: every weight once (layers, LoRA factors, tied head, one gathered row),
    the KV read of ctx - 1 cached positions and the write of the new one."""
    import synth
    wb = synth.weight_bytes(shape, lora_rank)
    kv = synth.kv_bytes_per_position(shape) * kv_elem_bytes // 4
    return wb["layers"] + wb["lora"] + wb["lm_head"] + wb["embed_row"] + kv * ctx


def make_decoder(wl, path, stream, dw, dl=None, kv_bf16=False):
    import torch
    import decoder_only_token_amd as qd
    cfg = qd.make_config(wl.shape, max_prefill=wl.max_prefill, lora_rank_max=wl.lora_rank,
                         decode_path=qd.QD_DECODE_PERSISTENT if path == "persistent" else qd.QD_DECODE_GRAPH,
                         kv_format=qd.QD_KV_BF16 if kv_bf16 else qd.QD_KV_F32)
    dec = qd.Decoder(cfg, stream.cuda_stream)
    dec.load_weights(dw)
    if dl is not None:
        dec.set_lora(dl, wl.lora_rank, wl.lora_alpha)
    torch.cuda.synchronize()
    return dec


def fill_to(dec, wl, stream, target):
    """Untimed: reset, the workload's prompt as one batched prefill, then
    batched prefills of random tokens until `target` positions are cached."""
    import synth
    import torch
    shape = wl.shape
    with torch.cuda.stream(stream):
        dec.reset_kv()
        prompt = synth.make_prompt(shape.vocab, min(wl.prompt_len, target))
        dec.prefill(prompt)
        at, k = len(prompt), 0
        while at < target:
            n = min(wl.max_prefill, target - at)
            dec.prefill(synth.make_prompt(shape.vocab, n, seed=100 + k))
            at += n
            k += 1
    dec.sync_token()
    assert dec.position == target


def decode_at_end(dec, wl, stream, steps, warmup, kv_elem_bytes=4):
    """`warmup` untimed and `steps` timed decode steps ending at the last
    cache position; HIP events on the library's stream bracket the timed steps."""
    import torch
    end = wl.shape.max_pos
    start = end - steps - warmup
    fill_to(dec, wl, stream, start)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            dec.decode_step()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(steps):
            dec.decode_step()
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    if dec.abandoned():
        raise RuntimeError("a persistent decode step was abandoned (device shared with other work)")
    ms = a.elapsed_time(b)
    ctx0 = start + warmup + 1  # context after the first timed step
    byts = [step_bytes(wl.shape, wl.lora_rank, ctx0 + i, kv_elem_bytes) for i in range(steps)]
    return {"steps": steps, "wall_s": wall, "event_ms": ms, "ctx_first": ctx0, "ctx_last": ctx0 + steps - 1,
            "bytes_per_step": sum(byts) / steps}


def verify_rate(dec, wl, stream, ms_rows=(4, 8, 16), reps=5):
    """Speculative verification at the end of the context: qd_verify of m rows
    then qd_rewind(m), so every call runs at the same context; the median time
    per call and the tokens/s it gives when every draft is accepted (m tokens
    per call)."""
    import numpy as np
    import synth
    import torch
    start = wl.shape.max_pos - 16 - 1
    fill_to(dec, wl, stream, start)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    out = {"context": start}
    with torch.cuda.stream(stream):
        for m in ms_rows:
            if m > wl.max_prefill:
                continue
            toks = synth.make_prompt(wl.shape.vocab, m, seed=300 + m)
            dts = []
            for r in range(reps + 1):
                torch.cuda.synchronize()
                a, b = ev(), ev()
                a.record(stream)
                dec.verify(toks)
                dec.rewind(m, int(toks[0]))
                b.record(stream)
                torch.cuda.synchronize()
                if r:
                    dts.append(a.elapsed_time(b))
            t = float(np.median(dts))
            out[f"m{m}"] = {"us_per_call": round(t * 1e3, 1), "tok_s_all_accepted": round(m / (t * 1e-3), 1)}
    return out


def multistep_rate(dec, wl, stream, n=16, batches=3):
    """qd_decode_steps with n tokens per call (one host synchronisation per
    call), `batches` timed calls after one untimed, ending at the last cache
    position; HIP events on the library's stream bracket the timed calls."""
    import torch
    end = wl.shape.max_pos
    fill_to(dec, wl, stream, end - n * (batches + 1))
    toks = torch.empty(n, dtype=torch.int32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    with torch.cuda.stream(stream):
        dec.decode_steps(n, tokens_out=toks)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        t0 = time.perf_counter()
        a.record(stream)
        for _ in range(batches):
            dec.decode_steps(n, tokens_out=toks)
            stream.synchronize()  # one host synchronisation per call
        b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    if dec.abandoned():
        raise RuntimeError("a persistent decode step was abandoned")
    steps = n * batches
    return {"tokens_per_call": n, "calls": batches, "tok_s": round(steps / wall, 2),
            "step_us": round(a.elapsed_time(b) * 1e3 / steps, 2),
            "note": "greedy; one launch per run of steps with one attention split count on the persistent "
                    "path, one launch per step on the graph path"}


def prefill_rate(dec, wl, stream, rows):
    """Median of 3 batched prefills of `rows` tokens from an empty cache; FLOPs
    are the algorithmic ones (2 per weight per row for the projections, the
    LoRA products, and 2 * 2 * d per visible key per q head for attention)."""
    import numpy as np
    import synth
    import torch
    shape = wl.shape
    toks = synth.make_prompt(shape.vocab, rows, seed=7)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    times = []
    with torch.cuda.stream(stream):
        for i in range(4):
            dec.reset_kv()
            a, b = ev(), ev()
            a.record(stream)
            dec.prefill(toks)
            b.record(stream)
            torch.cuda.synchronize()
            if i:
                times.append(a.elapsed_time(b))
    dec.sync_token()
    ms = float(np.median(times))
    H, d, I, L = shape.hidden, shape.head_dim, shape.intermediate, shape.n_layers
    nq, nkv = shape.n_q_heads, shape.n_kv_heads
    lin = (nq * d + 2 * nkv * d) * H + H * nq * d + 2 * I * H + H * I
    lora = wl.lora_rank * (2 * H + nq * d + nkv * d)
    proj = 2.0 * rows * (lin + lora) * L
    attn = 2.0 * 2.0 * d * nq * L * (rows * (rows + 1) / 2)
    return {"rows": rows, "ms": round(ms, 3), "tok_s": round(rows / (ms * 1e-3), 1),
            "projection_tflops": round(proj / (ms * 1e-3) / 1e12, 2),
            "attention_tflops": round(attn / (ms * 1e-3) / 1e12, 2),
            "mfma_util_lower_bound": round((proj + attn) / (ms * 1e-3) / (MFMA_PEAK_BF16_TFLOPS * 1e12), 4),
            "note": "whole prefill time (projections on the matrix cores, attention, norms, LM head row); "
                    "algorithmic FLOPs over the bf16 dense peak (the hi/lo input split issues each product twice)"}


def job_06b(stream, path, workload="qwen3-0.6b"):
    """qwen3-0.6b (or its Q8_0 form): jobs of reset + 5-token prefill + 128
    greedy decode steps (the configuration of the earlier measurements),
    decode roofline."""
    import numpy as np
    import synth
    import torch
    wl = synth.WORKLOADS[workload]
    dw = synth.make_weights_device(wl.shape)
    dec = make_decoder(wl, path, stream, dw)
    del dw
    prompt = synth.make_prompt(wl.shape.vocab, wl.prompt_len)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    dts = []
    with torch.cuda.stream(stream):
        for i in range(4):
            dec.reset_kv()
            dec.prefill(prompt)
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(wl.decode_steps):
                dec.decode_step()
            b.record(stream)
            torch.cuda.synchronize()
            if i:
                dts.append(a.elapsed_time(b))
    if dec.abandoned():
        raise RuntimeError("a persistent decode step was abandoned")
    dec.close()
    ms = float(np.median(dts))
    n = wl.decode_steps
    byts = sum(step_bytes(wl.shape, 0, wl.prompt_len + 1 + i) for i in range(n)) / n
    us = ms * 1e3 / n
    ach = byts / (us * 1e-6) / 1e9
    return {"workload": wl.name, "decode_path": path, "decode_tok_s": round(n / (ms * 1e-3), 1),
            "decode_step_us": round(us, 2), "bytes_per_step": round(byts),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(wl.name, path)}}


def job_q8(stream):
    """The Q8_0 weight format on qwen3-0.6b ("SuperKittens pull request #7"
    compares Q8_0 with fp16 weights on this model): the same decode job with
    Q8_0 and with bf16 projection weights, both on the per-operation graph
    (Q8_0 runs there only), and the ratio."""
    q8 = job_06b(stream, "graph", "qwen3-0.6b-q8_0")
    bf = job_06b(stream, "graph", "qwen3-0.6b")
    return {"q8_0": q8, "bf16": bf, "q8_0_over_bf16": round(q8["decode_tok_s"] / bf["decode_tok_s"], 3),
            "dtype": dtype_of(synth_shape("qwen3-0.6b-q8_0"), "graph")}


def synth_shape(name):
    import synth
    return synth.WORKLOADS[name].shape


def job_c4(stream, steps=20, warmup=5):
    """qwen2.5-3b-int4 (4096 positions): decode at the end of the context on
    the captured graph (its default path) and on the persistent step (with
    its measured traffic), each with its roofline."""
    import synth
    import torch
    wl = synth.WORKLOADS["qwen2.5-3b-int4"]
    dw = synth.make_weights_device(wl.shape)
    res = {}
    for path in ("graph", "persistent"):
        dec = make_decoder(wl, path, stream, dw)
        d = decode_at_end(dec, wl, stream, steps, warmup)
        dec.close()
        torch.cuda.synchronize()
        us = d["event_ms"] * 1e3 / steps
        ach = d["bytes_per_step"] / (us * 1e-6) / 1e9
        res[path] = {"decode_path": path, "decode_tok_s": round(steps / d["wall_s"], 2),
                     "decode_step_us": round(us, 2), "decode_context": [d["ctx_first"], d["ctx_last"]],
                     "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(ach / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic(wl.name, path),
                                  "kernel": ("k_decode_persistent (one launch = one decode step)"
                                             if path == "persistent" else "decode step (captured graph)")}}
    del dw
    torch.cuda.empty_cache()
    out = {"workload": wl.name}
    out.update(res["graph"])
    out["persistent"] = res["persistent"]
    return out


def job_kv_bf16(wl, stream, dw, dl, steps=20, warmup=5):
    """The headline workload with a bf16 KV cache (graph path): half the cache
    bytes; the rounding of keys and values is part of that model variant."""
    import torch
    dec = make_decoder(wl, "graph", stream, dw, dl, kv_bf16=True)
    d = decode_at_end(dec, wl, stream, steps, warmup, kv_elem_bytes=2)
    dec.close()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    us = d["event_ms"] * 1e3 / steps
    ach = d["bytes_per_step"] / (us * 1e-6) / 1e9
    return {"workload": wl.name, "kv_format": "bf16", "decode_path": "graph",
            "decode_tok_s": round(steps / d["wall_s"], 2), "decode_step_us": round(us, 2),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": f"decode step (captured graph); algorithmic bytes per step = {d['bytes_per_step']:.4g} "
                                   "(KV at 2 bytes per element)"}}


def cpu_baseline(wl, dw, dl, ctx):
    """The float64 oracle on a bounded sample of the timed step: one decode
    token at context `ctx`, on the model cut to 1 and to 4 layers (its KV cache
    filled with seeded random keys and values for ctx - 1 positions: the
    arithmetic does not depend on their values), plus the tied head; the
    36-layer time is t(1) + 35 (t(4) - t(1)) / 3 (three layers' difference, so
    that timing noise on the head does not swamp one layer's time).  Timed
    with all host threads and with one thread."""
    import dataclasses
    import numpy as np
    import synth
    from oracle import OracleModel
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    shape = wl.shape
    host = synth.device_to_host(dw, layers=[0, 1, 2, 3])
    lora = None
    if dl is not None:
        lora = [{k: v.cpu().numpy().view(np.uint16) for k, v in dl[i].items()} for i in range(4)]
    t_build = time.perf_counter()
    models = {}
    for nl in (1, 4):
        s = dataclasses.replace(shape, n_layers=nl)
        sub = {"embed": host["embed"], "final_norm": host["final_norm"], "layers": host["layers"][:nl]}
        models[nl] = OracleModel(s, sub, lora=lora[:nl] if lora else None, lora_alpha=wl.lora_alpha)
    t_build = time.perf_counter() - t_build
    rng = np.random.default_rng(11)

    def one_token(m):
        cache = m.new_cache(ctx)
        for li in range(m.shape.n_layers):
            cache.k[li][:ctx - 1] = rng.standard_normal((ctx - 1, shape.n_kv_heads, shape.head_dim))
            cache.v[li][:ctx - 1] = rng.standard_normal((ctx - 1, shape.n_kv_heads, shape.head_dim))
        cache.length = ctx - 1
        t = time.perf_counter()
        m.forward([1234], cache, logits_rows="last")
        return time.perf_counter() - t

    def estimate(reps):
        t1 = min(one_token(models[1]) for _ in range(reps))
        t4 = min(one_token(models[4]) for _ in range(reps))
        return t1 + (shape.n_layers - 1) * max(t4 - t1, 0.0) / 3, t1, t4

    cores = len(os.sched_getaffinity(0))
    t_all, t1, t4 = estimate(3)
    t_one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t_one = estimate(1)[0]
    return {"value": round(1.0 / t_all, 4), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "one_thread_tok_s": round(1.0 / t_one, 5) if t_one else None,
            "sample": f"{wl.name}: float64 numpy oracle, one decode token at context {ctx} on the model cut to "
                      f"1 and 4 layers (KV cache filled with seeded random values), 36-layer time = "
                      f"t1 + 35 (t4 - t1) / 3 = {t_all:.3f} s (t1 {t1:.3f} s, t4 {t4:.3f} s, best of 3; weight "
                      f"widening {t_build:.1f} s "
                      f"not counted); {cores} host threads"}


def dtype_of(shape, path):
    import synth
    if shape.weight_format == synth.W_Q8_0:
        w = "Q8_0 projection weights (int8 blocks of 32 x fp16 scales); codes widened in registers, f32 products (GEMV)"
    elif shape.weight_format == synth.W_INT4_G128:
        w = ("int4 group-128 projection weights x fp16 scales; " +
             ("int8 matrix-core products against the input split into three 7-bit pieces (error <= 2^-21 of the "
              "largest input of a wave's groups)" if path == "persistent" else
              "int8 matrix-core products against the input split into three 7-bit pieces (error <= 2^-20 of the "
              "row's largest input) for o_proj, gate/up and down, codes widened in registers with f32 products for "
              "q|k|v (GEMV); bf16 hi/lo matrix-core products (prefill)"))
    else:
        w = "bf16 weights, matrix-core GEMV with the input as bf16 hi/lo halves (16 significant bits)"
    return (w + "; bf16 tied embedding and LoRA factors; f32 accumulation, residual and KV cache" +
            ("; attention output and SwiGLU activations exchanged at 16 significant bits" if path == "persistent" else ""))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch
    import synth

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    # auto: the persistent step for bf16 weights without an adapter; the
    # captured graph otherwise (int4 single-row projections on the int8
    # matrix cores, split-K attention over every CU; Q8_0 runs only there)
    path = ("graph" if wl.lora_rank or wl.shape.weight_format != 0 else "persistent") if args.path == "auto" \
        else args.path
    dw = synth.make_weights_device(shape)
    dl = synth.make_lora_device(shape, wl.lora_rank) if wl.lora_rank else None
    torch.cuda.synchronize()
    dec = make_decoder(wl, path, stream, dw, dl)
    d = decode_at_end(dec, wl, stream, args.steps, args.warmup)
    us = d["event_ms"] * 1e3 / args.steps
    achieved = d["bytes_per_step"] / (us * 1e-6) / 1e9
    value = args.steps / d["wall_s"]
    out = {
        "metric": "decode tok/s + achieved HBM GB/s (% of peak); prefill tok/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["wall_s"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(shape, path),
        "data": "synthetic (seeded N(0,0.02) weights drawn on the GPU and rounded to bf16, uniform random token ids)",
        "config": {"workload": wl.name, "layers": shape.n_layers, "hidden": shape.hidden,
                   "heads": [shape.n_q_heads, shape.n_kv_heads], "intermediate": shape.intermediate,
                   "vocab": shape.vocab, "prompt_len": wl.prompt_len, "max_pos": shape.max_pos,
                   "decode_context": [d["ctx_first"], d["ctx_last"]], "global_batch": 1,
                   "parallelism": "single GPU", "decode_path": path,
                   "lora": {"rank": wl.lora_rank, "alpha": wl.lora_alpha} if wl.lora_rank else None},
        "decode_tok_s": round(args.steps / (d["event_ms"] * 1e-3), 2),
        "decode_step_us": round(us, 2),
        "decode_hbm_gbs_effective": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, path),
                     "kernel": ("k_decode_persistent (one launch = one decode step)" if path == "persistent"
                                else "decode step (captured graph of per-operation kernels)") +
                               f"; algorithmic bytes per step = {d['bytes_per_step']:.4g} (weights + LoRA + tied "
                               "head + one embedding row + KV read and write at the step's context)"},
    }
    if not args.only_decode and not args.no_extra:
        out["decode_steps_16"] = multistep_rate(dec, wl, stream)
        out["speculative_verify"] = verify_rate(dec, wl, stream)
        out["prefill_batched"] = prefill_rate(dec, wl, stream, wl.prompt_len)
    if not args.only_decode and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, dw, dl, shape.max_pos)
    if not args.only_decode and not args.no_extra and wl.name == "qwen2.5-3b-int4-lora":
        dec.close()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        out["kv_bf16"] = job_kv_bf16(wl, stream, dw, dl)
    dec.close()
    del dw, dl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.only_decode and not args.no_extra and wl.name != "qwen3-0.6b":
        out["qwen3_0_6b"] = job_06b(stream, "persistent" if args.path == "auto" else args.path)
    if not args.only_decode and not args.no_extra and wl.name != "qwen2.5-3b-int4":
        out["qwen2_5_3b_int4"] = job_c4(stream)
    if not args.only_decode and not args.no_extra:
        out["q8_0_qwen3_0_6b"] = job_q8(stream)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
