"""Benchmark of the forward selective scan on one MI355X.

One step = one forward scan call (softplus of delta, discretisation, the
recurrence, the C readout with the D skip, the silu gate, the bf16 store and
the final state) over the Mamba-2.8B-shaped layer workload (batch 4, D_inner
5120, N 16, L 2048, bf16 activations, fp32 parameters and state), with inputs
resident in HBM.  Prints one JSON line.

Inputs rotate over several buffer sets so that the 256 MB Infinity Cache
cannot hold a step's inputs from the previous step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
CUS, SIMDS, LANES, CLOCK_GHZ = 256, 4, 16, 2.4
VALU_PEAK_TSLOTS = CUS * SIMDS * LANES * CLOCK_GHZ / 1e3   # 39.32 T lane-slots/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2p8b_layer")
    ap.add_argument("--time-segments", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"))
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows are independent; see DESIGN.md for how it would shard).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    import selective_state_space_52_amd as m

    s = W.spec(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sets = []
    base = W.make_scan_inputs(s)
    for r in range(max(1, args.rotate)):
        if r == 0:
            inp = base
        else:  # distinct buffers, same distributions (different seed)
            inp = W.make_scan_inputs(W.spec(args.workload, seed=s.seed + 1000 * r))
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        d["out"] = torch.empty_like(d["u"])
        d["last"] = torch.empty(s.batch, s.dim, s.dstate, device=dev)
        sets.append(d)

    def step(i):
        d = sets[i % len(sets)]
        m.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                             z=d["z"], delta_bias=d["delta_bias"],
                             softplus=s.softplus, last_state=d["last"],
                             out=d["out"], time_segments=args.time_segments)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps

    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen,
                       torch.bfloat16 if s.io == "bf16" else torch.float32,
                       args.time_segments)
    nbytes = W.scan_bytes(s)
    gbs = nbytes / (ms * 1e-3) / 1e9
    gelem = s.state_elements / (ms * 1e-3) / 1e9
    # algorithmic VALU issue slots: per state element one multiply (Delta*A),
    # one exp (2 slots: v_exp_f32 issues at half rate), one multiply (Delta*u
    # times B), two fma (state update, C readout) = 6; per element the
    # softplus (~16), Delta*u, D skip, silu gate (~8) and bf16 conversions
    # (~4) = 30
    slots = s.state_elements * 6 + s.elements * 30
    achieved_tslots = slots / (ms * 1e-3) / 1e12

    traffic = None
    try:
        with open(args.traffic) as f:
            tr = json.load(f)
        key = "%s/%s" % (args.workload, plan["segments"])
        if key in tr:
            traffic = tr[key]
    except (OSError, ValueError):
        pass

    res = {
        "metric": "selective-scan fwd HBM GB/s (% of peak) + Gelem/s (B*L*D_inner*N)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if s.io == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": "%s: batch %d, D_inner %d, N %d, L %d, %s io, fp32 state"
                   % (s.name, s.batch, s.dim, s.dstate, s.seqlen, s.io),
                   "batch": s.batch, "d_inner": s.dim, "d_state": s.dstate,
                   "seq_len": s.seqlen, "plan": plan},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "gelem_per_s": round(gelem, 2),
        "roofline": {"bound": "alu", "achieved": round(achieved_tslots, 3),
                     "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                     "frac": round(achieved_tslots / VALU_PEAK_TSLOTS, 4),
                     "traffic": traffic},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(s, base, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_baseline(s, inp, seconds):
    """The fp64 oracle on the host cores, on a bounded sample of rows of the
    same workload (whole rows, all L timesteps), scaled to Gelem/s."""
    import oracle
    import numpy as np
    nth = oracle.default_threads()
    rows_total = s.batch * s.dim
    # grow the sample until it takes about `seconds`
    k = 64
    while True:
        sub = {key: v for key, v in inp.items()}
        b_idx = 0
        d_idx = slice(0, min(k, s.dim))
        sub = dict(u=inp["u"][b_idx:b_idx + 1, d_idx], delta=inp["delta"][b_idx:b_idx + 1, d_idx],
                   z=inp["z"][b_idx:b_idx + 1, d_idx], B=inp["B"][b_idx:b_idx + 1],
                   C=inp["C"][b_idx:b_idx + 1], A=inp["A"][d_idx], D=inp["D"][d_idx],
                   delta_bias=inp["delta_bias"][d_idx])
        conv = {key: oracle._f64(v) for key, v in sub.items()}
        t0 = time.perf_counter()
        oracle.scan(conv["u"], conv["delta"], conv["A"], conv["B"], conv["C"], D=conv["D"],
                    z=conv["z"], delta_bias=conv["delta_bias"], softplus=s.softplus,
                    nthreads=nth)
        dt = time.perf_counter() - t0
        rows = conv["u"].shape[1]
        if dt >= seconds or rows >= s.dim:
            break
        k = min(s.dim, max(2 * k, int(k * seconds / max(dt, 1e-3) * 1.1)))
    gelem = rows * s.seqlen * s.dstate / dt / 1e9
    return {"value": round(gelem, 4), "unit": "Gelem/s", "cores": nth, "kind": "oracle",
            "sample": "%d of %d rows (batch 0, channels 0..%d), all %d timesteps, %.1f s"
                      % (rows, rows_total, rows - 1, s.seqlen, dt)}


if __name__ == "__main__":
    main()
