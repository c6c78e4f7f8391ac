"""Benchmark: single-sequence decode (and prefill) of a Qwen3-style decoder on one MI355X.

One timed step = one whole generation job of the workload: reset the KV cache,
batched prefill of the prompt, then the workload's greedy decode steps, all
through the C ABI on one HIP stream, with weights and inputs resident in HBM.

Prints ONE JSON line.  `value` = generated tokens per second over the whole
job (prefill token + decode tokens); decode-only and prefill rates, the
effective HBM bandwidth and the dominant kernel's roofline fraction are
reported beside it.  The CPU oracle is timed on a bounded sample of the same
workload on the host cores (`cpu_baseline`).
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
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3-0.6b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-rows", type=int, default=512,
                    help="also time one batched prefill of this many random tokens (0: skip)")
    ap.add_argument("--cpu-sample-steps", type=int, default=128)
    ap.add_argument("--path", choices=["auto", "persistent", "graph"], default="auto",
                    help="decode step as one persistent kernel, or as per-operation kernels in a hipGraph "
                         "(auto: persistent where the model allows it: bf16 weights, no adapter)")
    ap.add_argument("--decode-steps", type=int, default=0,
                    help="decode steps per job (0: the workload's own count)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 launches): the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


# Sources of the persistent decode kernel: HBM traffic measured with counters
# is reported only while these are unchanged since the counters were taken.
KERNEL_SOURCES = ["decoder_only_token_amd/csrc/persist.hip", "decoder_only_token_amd/csrc/persist.h",
                  "decoder_only_token_amd/csrc/common.h"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the persistent decode kernel from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel factor),
    or None when there is none for this workload or the kernel has changed since."""
    path = os.path.join(ROOT, "profiles", f"k_decode_persistent.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
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


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(wl, weights, prompt, n_steps, min_seconds=10.0, max_jobs=8):
    """Time the oracle (as it stands) on the host: jobs of prompt + n_steps
    incremental greedy steps, repeated until about min_seconds of CPU work."""
    from oracle import OracleModel, argmax_lowest
    t_build = time.perf_counter()
    m = OracleModel(wl.shape, weights)
    t_build = time.perf_counter() - t_build
    toks, jobs = 0, 0
    t0 = time.perf_counter()
    while jobs < max_jobs and (jobs == 0 or time.perf_counter() - t0 < min_seconds):
        cache = m.new_cache(len(prompt) + n_steps + 1)
        logits = m.forward(prompt, cache, logits_rows="last")[-1]
        toks += 1
        for _ in range(n_steps):
            logits = m.forward([argmax_lowest(logits)], cache, logits_rows="last")[-1]
            toks += 1
        jobs += 1
    dt = time.perf_counter() - t0
    cores = blas_threads()
    return {"value": toks / dt, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{wl.name}: float64 numpy oracle, {jobs} job(s) of prefill {len(prompt)} tokens + {n_steps} "
                      f"greedy decode steps with its own KV cache ({toks} tokens in {dt:.1f} s; weight widening "
                      f"{t_build:.1f} s not counted); {cores} BLAS threads"}


def measure_long_prefill(dec, stream, shape, wl, args):
    """Time a batched prefill of args.prefill_rows seeded random tokens on the
    same model (the projections run on the matrix cores).  FLOP counts are the
    algorithmic ones: 2 per weight per row for the projections, plus the causal
    attention products (2 * 2 * d per visible key per q head)."""
    import numpy as np
    import torch
    import synth
    n = args.prefill_rows
    if n > wl.max_prefill or n > shape.max_pos:
        return None
    toks = synth.make_prompt(shape.vocab, n, seed=7)
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
    proj = 2.0 * n * lin * L
    attn = 2.0 * 2.0 * d * nq * L * (n * (n + 1) / 2)
    return {"rows": n, "ms": round(ms, 3), "tok_s": round(n / (ms * 1e-3), 1),
            "projection_tflops": round(proj / (ms * 1e-3) / 1e12, 2),
            "mfma_util_lower_bound": round(proj / (ms * 1e-3) / (MFMA_PEAK_BF16_TFLOPS * 1e12), 4),
            "note": "whole prefill time (projections, attention, norms, LM head row); projection FLOPs "
                    "counted once although the hi/lo input split issues each product twice"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import numpy as np
    import torch
    import synth
    import decoder_only_token_amd as qd

    wl = synth.WORKLOADS[args.workload]
    shape = wl.shape
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    weights = synth.make_weights(shape)
    prompt = synth.make_prompt(shape.vocab, wl.prompt_len)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()  # noqa: E731
    dw = {"embed": to_dev(weights["embed"]), "final_norm": to_dev(weights["final_norm"]),
          "layers": [{k: to_dev(v) for k, v in lw.items()} for lw in weights["layers"]]}
    torch.cuda.synchronize()
    if args.path == "auto":
        args.path = "persistent" if shape.weight_format == synth.W_BF16 and not wl.lora_rank else "graph"
    path = qd.QD_DECODE_PERSISTENT if args.path == "persistent" else qd.QD_DECODE_GRAPH
    dec = qd.Decoder(qd.make_config(shape, max_prefill=wl.max_prefill, lora_rank_max=wl.lora_rank,
                                    decode_path=path), stream.cuda_stream)
    dec.load_weights(dw)
    del dw
    if wl.lora_rank:
        lora = synth.make_lora(shape, wl.lora_rank)
        dl = [{k: to_dev(v) for k, v in lw.items()} for lw in lora]
        torch.cuda.synchronize()
        dec.set_lora(dl, wl.lora_rank, wl.lora_alpha)
        del dl
    torch.cuda.synchronize()
    n_dec = args.decode_steps or wl.decode_steps
    sampling = (qd.make_sampling(wl.temperature, wl.top_k, wl.top_p, synth.SEED_SAMPLING)
                if wl.temperature > 0 else None)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def job(marks=None, samp=None):
        dec.reset_kv()
        if marks:
            marks[0].record(stream)
        dec.prefill(prompt, sampling=samp)
        if marks:
            marks[1].record(stream)
        for _ in range(n_dec):
            dec.decode_step(sampling=samp)
        if marks:
            marks[2].record(stream)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            job()
        torch.cuda.synchronize()
        marks = [[ev(), ev(), ev()] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            job(marks[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    dec.sync_token()  # raises if any decode step was abandoned
    sampled = None
    if sampling is not None:
        with torch.cuda.stream(stream):
            m = [ev(), ev(), ev()]
            job(m, sampling)
            torch.cuda.synchronize()
        dec.sync_token()
        s_ms = m[1].elapsed_time(m[2])
        sampled = {"temperature": wl.temperature, "top_k": wl.top_k, "top_p": wl.top_p, "seed": synth.SEED_SAMPLING,
                   "decode_tok_s": round(n_dec / (s_ms * 1e-3), 2), "decode_step_us": round(s_ms * 1e3 / n_dec, 2),
                   "note": "one job with on-GPU top-k / temperature / top-p draws (greedy is the headline)"}
    long_prefill = measure_long_prefill(dec, stream, shape, wl, args) if args.prefill_rows else None
    prefill_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / args.steps
    decode_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_job = 1 + n_dec
    value = tokens_per_job * args.steps / wall

    kvp = synth.kv_bytes_per_position(shape)
    # algorithmic HBM bytes of one decode step at context c: all weights once
    # (layers + tied head + one gathered row), KV read for c positions, KV write of one position
    ctx0 = wl.prompt_len
    wb = synth.weight_bytes(shape, wl.lora_rank)
    dec_bytes = sum((wb["layers"] + wb["lora"] + wb["lm_head"] + wb["embed_row"]) + kvp * (ctx0 + i + 1)
                    for i in range(n_dec))
    decode_step_us = decode_ms * 1e3 / n_dec
    achieved = dec_bytes / n_dec / (decode_step_us * 1e-6) / 1e9
    traffic = measured_traffic(wl.name) if args.path == "persistent" else None
    out = {
        "metric": "decode tok/s + achieved HBM GB/s (% of peak); prefill tok/s, 1 MI355X",
        "value": round(value, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int4-g128 projection weights with fp16 scales, bf16 tied embedding"
                  if shape.weight_format == synth.W_INT4_G128 else "bf16 weights") +
                 ", f32 activations/accumulation/KV",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, uniform random prompt ids)",
        "config": {"workload": wl.name, "model": shape.name, "layers": shape.n_layers, "hidden": shape.hidden,
                   "heads": [shape.n_q_heads, shape.n_kv_heads], "vocab": shape.vocab,
                   "prompt_len": wl.prompt_len, "decode_steps": n_dec, "global_batch": 1,
                   "parallelism": "single GPU", "decode_path": args.path,
                   "lora": {"rank": wl.lora_rank, "alpha": wl.lora_alpha} if wl.lora_rank else None},
        "decode_tok_s": round(n_dec / (decode_ms * 1e-3), 2),
        "decode_step_us": round(decode_step_us, 2),
        "prefill_tok_s": round(wl.prompt_len / (prefill_ms * 1e-3), 2),
        "prefill_ms": round(prefill_ms, 3),
        "decode_hbm_gbs_effective": round(achieved, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": ("k_decode_persistent (one launch = one decode step)" if args.path == "persistent"
                                else "decode step (captured graph of per-operation kernels)") +
                               "; algorithmic bytes = weights + KV read + KV write"},
    }
    if long_prefill:
        out["prefill_batched"] = long_prefill
    if sampled:
        out["sampled"] = sampled
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, weights, prompt, args.cpu_sample_steps)
    dec.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
