"""Phase trace of one persistent decode step: where a layer's time goes.

    python -m decoder_only_token_amd.phase_trace --workload qwen3-0.6b --ctx 133

Fills the cache of the named synthetic workload (weights drawn on the GPU) to
`ctx` positions, runs three untimed steps and then one traced step, and
prints from the per-CU stamps (100 MHz real-time counter, `qd_get_phase_trace`):

* the CUs of each role;
* per phase, the critical hop (the producing role's last publish -> this
  role's last input ready) and the compute time (last input ready -> last
  outputs published), which add up to the layer period;
* each consuming CU's hop (producer's last publish -> its own input ready),
  its median, its minimum (the floor of a store -> visible -> seen round
  trip in this step) and its median split by whether the consuming CU sits on
  the same XCD as that last producer (workgroups are dealt to the 8 XCDs round
  robin, so XCD = workgroup index mod 8).

Diagnostics only; the decode step itself does not depend on this module.
"""
from __future__ import annotations

import argparse
import os
import sys

ROLES = ["qkv", "attn", "o_proj", "gate_up", "down"]
N_XCD = 8


def trace_step(workload: str, ctx: int, cus: int = 0):
    import numpy as np
    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import synth
    import decoder_only_token_amd as qd
    wl = synth.WORKLOADS[workload]
    shape = wl.shape
    if cus:
        os.environ["QD_PERSIST_CUS"] = str(cus)
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    dw = synth.make_weights_device(shape)
    cfg = qd.make_config(shape, max_prefill=wl.max_prefill, decode_path=qd.QD_DECODE_PERSISTENT)
    dec = qd.Decoder(cfg, stream.cuda_stream)
    dec.load_weights(dw)
    del dw
    dec.reset_kv()
    at = 0
    while at < ctx:
        n = min(wl.max_prefill, ctx - at)
        dec.prefill(synth.make_prompt(shape.vocab, n, seed=at))
        at += n
    for _ in range(3):
        dec.decode_step()
    dec.enable_phase_trace(True)
    dec.decode_step()
    tr = dec.get_phase_trace().astype(np.int64)
    dec.close()
    return shape, tr


def summarize(shape, tr) -> list:
    """Per-phase budget of the interior layers.  For phase r of layer l, with
    P = the last publish (slot 3) of the producing phase and R, Q = the last
    input-ready (slot 1) and last publish of this phase over its CUs:
    critical hop = R - P, compute = Q - R.  Their sum over the five phases of a
    layer telescopes to the layer period (down's last publish of layer l - 1 to
    that of layer l).  A CU's hop is its own ready stamp minus P; its
    minimum over CUs and layers is the hop floor seen in this step."""
    import numpy as np
    L = shape.n_layers
    ncu = tr.shape[0]
    role_of = np.full(ncu, -1)
    for cu in range(ncu):
        for r in range(5):
            if tr[cu, 8 * r + 0] or tr[cu, 8 * r + 1]:
                role_of[cu] = r
    cus = [np.nonzero(role_of == r)[0] for r in range(5)]
    out = ["CUs per role: " + ", ".join(f"{ROLES[r]} {len(cus[r])}" for r in range(5))]
    us = lambda t: float(t) / 100.0  # noqa: E731
    last = lambda p, r, k: max(tr[cu, 8 * p + k] for cu in cus[r])  # noqa: E731
    crit = {r: [] for r in range(5)}
    comp = {r: [] for r in range(5)}
    hops = {r: [] for r in range(5)}
    same = {r: [] for r in range(5)}
    cross = {r: [] for r in range(5)}
    period = []
    for l in range(1, L - 1):  # interior layers
        for r in range(5):
            p = 5 * l + r
            pr = (r - 1) % 5
            pp = p - 1  # the producing phase (qkv: down of the layer before)
            ppub = [tr[cu, 8 * pp + 3] for cu in cus[pr]]
            P = max(ppub)
            lastcu = cus[pr][int(np.argmax(ppub))]
            R, Q = last(p, r, 1), last(p, r, 3)
            crit[r].append(us(R - P))
            comp[r].append(us(Q - R))
            for cu in cus[r]:
                h = us(tr[cu, 8 * p + 1] - P)
                hops[r].append(h)
                (same if cu % N_XCD == lastcu % N_XCD else cross)[r].append(h)
        period.append(us(last(5 * l + 4, 4, 3) - last(5 * l - 1, 4, 3)))
    med = lambda v: float(np.median(v)) if len(v) else float("nan")  # noqa: E731
    out.append(f"{'phase':8} {'crit hop':>8} {'compute':>8} {'hop med':>8} {'same XCD':>9} "
               f"{'cross XCD':>9} {'hop min':>8}   (us)")
    tc = th = tf = 0.0
    for r in range(5):
        tc += med(comp[r])
        th += med(crit[r])
        tf += min(hops[r])
        out.append(f"{ROLES[r]:8} {med(crit[r]):8.2f} {med(comp[r]):8.2f} {med(hops[r]):8.2f} "
                   f"{med(same[r]):9.2f} {med(cross[r]):9.2f} {min(hops[r]):8.2f}")
    out.append(f"layer period: median {med(period):.2f} us; sum of the medians: critical hops {th:.2f} "
               f"+ compute {tc:.2f} = {th + tc:.2f} us")
    out.append(f"with every hop at this step's floor: {tf:.2f} + {tc:.2f} = {tf + tc:.2f} us per layer")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="qwen3-0.6b")
    ap.add_argument("--ctx", type=int, default=133)
    ap.add_argument("--cus", type=int, default=0, help="fewer workgroups than CUs (0: one per CU)")
    args = ap.parse_args()
    shape, tr = trace_step(args.workload, args.ctx, args.cus)
    print(f"workload {args.workload}, traced decode step at context {args.ctx + 4}")
    for line in summarize(shape, tr):
        print(line)


if __name__ == "__main__":
    main()
