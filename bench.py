"""Benchmark of the selective-scan hot path on one MI355X.

One step = one s6_scan_fwd over the Mamba-3B-shaped layer (batch 8,
D 5120, N 16, L 2048, bf16 inputs, fp32 state and output, SiLU gate, final
state returned), inputs already resident in device memory.  The decode step
(s6_state_update) is measured in the same run on its own workload (batch 256,
D 5120, N 16, 1024 single-token steps) and reported under "decode".

Prints ONE JSON line.  `value` is the scan's algorithmic bytes per second
(GB/s); `roofline` relates the scan kernel's rate to HBM peak; `cpu_baseline`
is the fp64 CPU oracle timed on a bounded sample of the same workload.
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


def scan_bytes(w, in_bytes, h0=False, h_last=True):
    """Algorithmic bytes of one scan: x, delta (and z) per token-channel,
    y (fp32) per token-channel, B and C per (batch, state, token), A and D
    once, optional h0 / h_last."""
    T = w.batch * w.dim * w.seqlen
    ntens = 3 if w.gate else 2
    b = T * (ntens * in_bytes + 4)
    b += 2 * w.batch * w.dstate * w.seqlen * in_bytes
    b += 4 * w.dim * w.dstate + 4 * w.dim
    if h0:
        b += 4 * w.batch * w.dim * w.dstate
    if h_last:
        b += 4 * w.batch * w.dim * w.dstate
    return b


def decode_step_bytes(batch, dim, N, in_bytes, gate=True):
    """One decode token: h read and written (fp32), x, delta (, z) in, y out
    (fp32) per channel; B, C per (batch, state); A and D once."""
    per = 2 * 4 * N + (3 if gate else 2) * in_bytes + 4
    return batch * dim * per + 2 * batch * N * in_bytes + 4 * dim * N + 4 * dim


def bench_scan(w, steps, warmup):
    import torch
    from selective_state_space_63_amd import s6, synth
    inp = synth.device_full(w)
    y = torch.empty((w.batch, w.dim, w.seqlen), device="cuda", dtype=torch.float32)
    hl = torch.empty((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)

    def step():
        s6.scan_fwd(inp["x"], inp["delta"], inp["A"], inp["Bm"], inp["Cm"], D=inp["Dskip"], z=inp["z"],
                    return_last_state=True, y=y, h_last=hl)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()  # the library launches on this stream
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    return inp, ms, wall


def bench_decode(steps_total, warmup):
    import torch
    from selective_state_space_63_amd import s6, synth
    w = synth.WORKLOADS["decode"]
    S = min(steps_total, w.seqlen)
    inp = synth.device_full(w)
    # per-step inputs laid out (S, batch, D) / (S, batch, N), contiguous per step
    x = inp["x"][..., :S].permute(2, 0, 1).contiguous()
    dl = inp["delta"][..., :S].permute(2, 0, 1).contiguous()
    z = inp["z"][..., :S].permute(2, 0, 1).contiguous()
    Bm = inp["Bm"][..., :S].permute(2, 0, 1).contiguous()
    Cm = inp["Cm"][..., :S].permute(2, 0, 1).contiguous()
    del inp["x"], inp["delta"], inp["z"]
    h = torch.zeros((w.batch, w.dim, w.dstate), device="cuda", dtype=torch.float32)
    y = torch.empty((w.batch, w.dim), device="cuda", dtype=torch.float32)

    def run(n):
        for s in range(n):
            s6.state_update(h, x[s], dl[s], inp["A"], Bm[s], Cm[s], D=inp["Dskip"], z=z[s], y=y)

    run(min(warmup, S))
    torch.cuda.synchronize()
    h.zero_()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    run(S)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    upd = w.batch * w.dim * w.dstate * S
    byts = decode_step_bytes(w.batch, w.dim, w.dstate, 2) * S
    return {
        "workload": w.name, "steps": S, "ms_total": round(ms, 3), "us_per_step": round(1e3 * ms / S, 2),
        "state_updates_per_s": upd / (ms * 1e-3), "token_steps_per_s": w.batch * S / (ms * 1e-3),
        "effective_GBps": byts / (ms * 1e-3) / 1e9,
        "note": "plain launches, state resident in device memory (fits the 256 MB Infinity Cache)",
    }


def cpu_baseline(w, inp, budget_s=6.0):
    """The fp64 oracle on whole batch rows of the same inputs, one row at a
    time until `budget_s` of wall time is spent (at least one row)."""
    import numpy as np
    import torch
    from oracle.oracle import Oracle
    o = Oracle()

    def h64(t):
        return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)

    A = h64(inp["A"])
    Dk = h64(inp["Dskip"])
    done_tc = 0
    spent = 0.0
    rows = 0
    for b in range(w.batch):
        args = dict(x=h64(inp["x"][b:b + 1]), delta=h64(inp["delta"][b:b + 1]), A=A,
                    Bm=h64(inp["Bm"][b:b + 1]), Cm=h64(inp["Cm"][b:b + 1]), Dskip=Dk,
                    z=h64(inp["z"][b:b + 1]))
        t0 = time.perf_counter()
        o.scan(**args)
        spent += time.perf_counter() - t0
        done_tc += w.dim * w.seqlen
        rows += 1
        if spent >= budget_s:
            break
    frac = rows / w.batch
    gbs = scan_bytes(w, 2) * frac / spent / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": o.num_threads(), "kind": "oracle",
            "sample": f"{rows} of {w.batch} batch rows (all {w.dim} channels x {w.seqlen} tokens each), "
                      f"{spent:.2f} s wall; {done_tc / spent:.3e} token-channels/s",
            "token_channels_per_s": done_tc / spent}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="m3b")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the scan has no cross-GPU step); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    from selective_state_space_63_amd import s6, synth
    s6.load_library()
    w = synth.WORKLOADS[args.workload]
    in_bytes = 2 if w.dtype == synth.BF16 else 4
    print(f"[bench] scan {w.name}: warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    inp, ms, wall = bench_scan(w, args.steps, args.warmup)
    byts = scan_bytes(w, in_bytes, h_last=True)
    gbs = byts / (ms * 1e-3) / 1e9
    tc = w.batch * w.dim * w.seqlen
    out = {
        "metric": "selective-scan fwd GB/s and % of HBM peak; decode state-updates/s",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in / f32 state and out" if in_bytes == 2 else "f32",
        "data": "synthetic (seeded, device-generated)",
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "dstate": w.dstate,
                   "seqlen": w.seqlen, "gate": w.gate, "final_state": True,
                   "algorithmic_bytes": byts},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "token_channels_per_s": tc / (ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_decode:
        print("[bench] decode", file=sys.stderr, flush=True)
        out["decode"] = bench_decode(args.decode_steps, args.warmup)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
