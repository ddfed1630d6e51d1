"""Benchmark of the forward selective scan on one MI355X.

One step = one forward scan call -- softplus of delta, discretisation, the
recurrence, the C readout with the D skip, the silu gate, the bf16 store and
the final state -- over the Mamba-2.8B-shaped layer workload (batch 4, D_inner
5120, N 16, L 2048, bf16 activations, fp32 parameters and state), with every
input already resident in HBM.  Rank 0 prints one JSON line.

Inputs rotate over several buffer sets so that the 256 MB Infinity Cache does
not hold a step's inputs from the step before.  The decode step (256 sequences
x D_inner 5120, N 16, 1000 steps) is reported beside it in "decode".

Other modes (used to produce the summaries under profiles/):
  --copy-calibration      time torch's copy of a 1 GiB buffer (the plain copy
                          kernel that scales the FETCH_SIZE/WRITE_SIZE counters)
  --rocprof-summary DIR   print per-kernel statistics of a rocprofv3 database
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TF = 2500.0     # MI355X dense bf16 matrix peak, TFLOP/s
CUS, SIMDS, LANES, CLOCK_GHZ = 256, 4, 16, 2.4
# fp32 VALU issue: one wave64 instruction per SIMD per 4 clocks = 16 lanes/clk
VALU_PEAK_TSLOTS = CUS * SIMDS * LANES * CLOCK_GHZ / 1e3   # 39.32 T lane-slots/s
# v_exp_f32 issues at half the fma rate (measured on the MI355X: 26.6 vs 54.8
# lane-ops per CU per clock), so the chip's exp peak is half the VALU peak
EXP_PEAK_T = VALU_PEAK_TSLOTS / 2                          # 19.66 T exp/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_main_traffic.json")
# the sources the forward scan kernel is built from (the traffic record is
# tied to them)
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_52_amd", "csrc", f)
                  for f in ("scan_fwd_impl.h", "scan_fwd.hip", "scan_fwd_n16.hip",
                            "scan_common.h", "dev_math.h")]

# Algorithmic VALU issue slots of the scan (fp32, one lane = one slot; a
# transcendental occupies two slots because v_exp/v_log/v_rcp issue at half
# rate).  Per state element: Delta*A (1), exp (2), Delta*u times B (1), the
# state fma (1), the C readout fma (1).  Per element: delta + bias (1),
# softplus = exp + log1p (2 + 2 + 3), Delta*u (1), D skip fma (1),
# silu = exp + reciprocal (2 + 2 + 2), gate multiply (1).
SLOTS_PER_STATE_ELEM = 6
SLOTS_PER_ELEM = 18
# The backward, counted the same way for the algorithm itself (one forward
# sweep keeping h_t, one reverse sweep), not for the kernel's recompute.  Per
# state element: the forward recurrence (5) and the C readout for dz (1); in
# reverse g += dy C, dy h (dC term), g Delta u (dB term), sum g B, g e, (g e)
# h_prev, sum A (g e h_prev), dA accumulate (8); one add each for the
# channel sums of dB and dC (2).  Per element: delta + bias (1), softplus
# (9), sigmoid of delta + bias (6), Delta*u (1), sigmoid of z (6),
# dy = dout z sigmoid(z) (2), dout silu'(z) (4), du (2), dDelta (1), ddelta
# (1), dz (2), dD and dbias accumulates (2).
BWD_SLOTS_PER_STATE_ELEM = 16
BWD_SLOTS_PER_ELEM = 37
# The width-4 causal conv in the fused path adds per element: 4 fmas and
# silu = exp + reciprocal (2 + 2) + 3, i.e. 11 slots.
CONV_SLOTS_PER_ELEM = 11


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2p8b_layer")
    ap.add_argument("--dstate", type=int, default=0,
                    help="override the workload's state size (0: keep it)")
    ap.add_argument("--time-segments", type=int, default=0)
    ap.add_argument("--rotate", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--bwd-time-segments", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-mamba2", action="store_true")
    ap.add_argument("--only-mamba2", action="store_true",
                    help="run the Mamba-2 scan leg alone (profiling runs)")
    ap.add_argument("--mamba2-traffic-record", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--mamba2-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=5.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--rocprof-summary", default=None)
    ap.add_argument("--traffic-record", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles made and read through the HIP runtime directly (the
    scan library records them around its main kernel; torch's Event objects
    refuse to time events that torch did not record itself)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        h = self.ct.c_void_p()
        if self.hip.hipEventCreate(self.ct.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a, b):
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return ms.value

    def destroy(self, h):
        self.hip.hipEventDestroy(h)


MAMBA2_SOURCES = [os.path.join(ROOT, "selective_state_space_52_amd", "csrc", f)
                  for f in ("mamba2.hip", "dev_math.h")]
MAMBA2_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mamba2_traffic.json")


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, plan: dict):
    """HBM bytes per forward call (all its kernels; the timed main kernel's
    window holds all of them but the B/C pack) from the committed counter
    summary, or None when it is missing or was taken on another version of
    the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    rec = tr.get(workload)
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    if rec.get("segments") != plan["segments"]:
        return None
    return rec.get("hbm_bytes_per_call")


def main():
    args = parse()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.traffic_record:
        traffic_record(args.workload, args.time_segments, *args.traffic_record)
        return
    if args.mamba2_traffic_record:
        mamba2_traffic_record(*args.mamba2_traffic_record)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the scan's rows are independent, so a "
              "multi-GPU run would shard them with no exchange, and this library "
              "has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import workloads as W
    import selective_state_space_52_amd as m

    if args.only_mamba2:
        print(json.dumps({"mamba2": bench_mamba2(torch, W, m, torch.device("cuda:0"),
                                                 args.mamba2_steps)}), flush=True)
        return
    over = {"dstate": args.dstate} if args.dstate else {}
    s = W.spec(args.workload, **over)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    io = torch.bfloat16 if s.io == "bf16" else torch.float32
    sets = []
    base = W.make_scan_inputs(s)
    for r in range(max(1, args.rotate)):
        inp = base if r == 0 else W.make_scan_inputs(
            W.spec(args.workload, seed=s.seed + 1000 * r, **over))
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
    # pass 1: the K timed steps as a caller runs them (no timing hook)
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
    # pass 2: the same steps with HIP events around the main scan kernel
    hev = HipEvents()
    pairs = [(hev.create(), hev.create()) for _ in range(args.steps)]
    for i in range(args.steps):
        m.set_scan_timing_events(*pairs[i])     # main scan kernel of this step
        step(i)
    torch.cuda.synchronize()
    m.set_scan_timing_events(None, None)
    per_step = sorted(hev.elapsed_ms(a, b) for a, b in pairs)
    main_ms = sum(per_step) / args.steps
    for a, b in pairs:
        hev.destroy(a)
        hev.destroy(b)

    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen, io, args.time_segments)
    nbytes = W.scan_bytes(s)
    gbs = nbytes / (ms * 1e-3) / 1e9
    gelem = s.state_elements / (ms * 1e-3) / 1e9
    slots = s.state_elements * SLOTS_PER_STATE_ELEM + s.elements * SLOTS_PER_ELEM
    achieved = slots / (main_ms * 1e-3) / 1e12
    traffic = load_traffic(args.workload, plan)

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
        "config": {"workload": "%s: batch %d, D_inner %d, N %d, L %d, %s activations, "
                               "fp32 A/D/delta_bias/state" % (s.name, s.batch, s.dim,
                                                              s.dstate, s.seqlen, s.io),
                   "batch": s.batch, "d_inner": s.dim, "d_state": s.dstate,
                   "seq_len": s.seqlen, "algorithmic_bytes": nbytes,
                   "plan": plan},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "gelem_per_s": round(gelem, 2),
        "roofline": {"bound": "alu", "achieved": round(achieved, 3),
                     "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                     "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
                     "traffic": traffic,
                     "kernel": "scan_kernel (main pass)",
                     "kernel_ms": round(main_ms, 5),
                     "kernel_ms_median": round(per_step[len(per_step) // 2], 5),
                     "kernel_ms_min": round(per_step[0], 5)},
        "exp_rate": {"achieved": round(s.state_elements / (main_ms * 1e-3) / 1e12, 3),
                     "peak": round(EXP_PEAK_T, 3), "unit": "T exp/s",
                     "frac": round(s.state_elements / (main_ms * 1e-3) / 1e12 / EXP_PEAK_T, 4)},
        "wall_s": round(wall, 3),
        "software": software(torch),
    }
    if not args.no_backward and s.dstate <= 32:   # the backward takes N <= 32
        res["backward"] = bench_backward(torch, W, m, dev, s, sets, hev,
                                         args.backward_steps,
                                         args.bwd_time_segments)
    if not args.no_conv:
        res["conv"] = bench_conv(torch, W, m, dev, s, sets, hev, ms)
    if not args.no_decode:
        res["decode"] = bench_decode(torch, W, m, dev, args.decode_steps)
    if not args.no_mamba2:
        res["mamba2"] = bench_mamba2(torch, W, m, dev, args.mamba2_steps)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(s, base, args.cpu_seconds, nbytes)
    print(json.dumps(res), flush=True)


def _time(torch, stream, fn, steps, warmup=3):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def mamba2_flops(s) -> float:
    """Algorithmic matrix flops of the chunked form (64-step chunks), counting
    each fp32 product once (not its hi/lo halves): per chunk, the causal half
    of C B^T (Q^2 N) and of (L o C B^T) X (Q^2 P), C H^T and the state
    update (2 Q N P each)."""
    Q = 64
    chunks = -(-s.seqlen // Q)
    per = Q * Q * s.dstate + Q * Q * s.headdim + 4 * Q * s.dstate * s.headdim
    return float(s.batch * s.nheads * chunks * per)


def bench_mamba2(torch, W, m, dev, steps=20):
    """The Mamba-2 block's scan (chunked matrix form on the matrix cores) on
    the Mamba-2-2.7B-shaped layer, 3 rotating input sets, against the
    selective scan of the same recurrence with A and the step expanded per
    channel."""
    s = W.spec("mamba2_2p7b_layer")
    stream = torch.cuda.current_stream(dev)
    sets = []
    for r in range(3):
        inp = W.make_mamba2_inputs(W.spec(s.name, seed=s.seed + 1000 * r))
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        d["last"] = torch.empty(s.batch, s.dim, s.dstate, device=dev)
        d["out"] = torch.empty_like(d["x"])
        sets.append(d)

    def call(i):
        d = sets[i % len(sets)]
        m.mamba2_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                          dt_bias=d["dt_bias"], softplus=s.softplus,
                          last_state=d["last"], out=d["out"])
    ms = _time(torch, stream, call, steps)
    d = sets[0]
    P = s.headdim
    gen = dict(u=d["x"].reshape(s.batch, s.seqlen, s.dim),
               delta=d["dt"].repeat_interleave(P, dim=2).contiguous(),
               A=d["A"].repeat_interleave(P)[:, None].expand(s.dim, s.dstate).contiguous(),
               D=d["D"].repeat_interleave(P).contiguous(),
               bias=d["dt_bias"].repeat_interleave(P).contiguous(),
               z=d["z"].reshape(s.batch, s.seqlen, s.dim),
               B=d["B"][:, :, 0].contiguous(), C=d["C"][:, :, 0].contiguous())
    gen_out = torch.empty_like(gen["u"])

    def general(i):
        m.selective_scan_fwd(gen["u"], gen["delta"], gen["A"], gen["B"], gen["C"],
                             D=gen["D"], z=gen["z"], delta_bias=gen["bias"],
                             softplus=s.softplus, last_state=d["last"], out=gen_out,
                             layout="bld")
    gen_ms = _time(torch, stream, general, max(3, steps // 4))
    nbytes = W.mamba2_bytes(s)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = mamba2_flops(s) / (ms * 1e-3) / 1e12
    return {"workload": "%s: batch %d, L %d, %d heads x %d channels, N %d, %d group(s), "
                        "bf16 activations, fp32 state" % (s.name, s.batch, s.seqlen,
                                                           s.nheads, s.headdim, s.dstate,
                                                           s.ngroups),
            "ms_per_step": round(ms, 5), "steps": steps,
            "algorithmic_bytes": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": load_mamba2_traffic(), "kernel": "mamba2_scan_kernel"},
            "mfma": {"achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TF, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TF, 4),
                     "algorithmic_flops": mamba2_flops(s)},
            "selective_scan_same_recurrence_ms": round(gen_ms, 5),
            "speedup_vs_selective_scan": round(gen_ms / ms, 2)}


def bench_conv(torch, W, m, dev, s, sets, hev, scan_ms, steps=20):
    """The causal conv (width 4, silu) ahead of the scan on the same workload:
    the standalone conv kernel (HBM-bound) and the conv fused into the scan's
    load stage, against running the two one after the other."""
    stream = torch.cuda.current_stream(dev)
    cps = [{k: v.to(dev) for k, v in
            W.make_conv_params(W.spec(s.name, seed=s.seed + 1000 * r, dstate=s.dstate)).items()}
           for r in range(len(sets))]
    u_bufs = [torch.empty_like(d["u"]) for d in sets]

    def conv(i):
        d, c = sets[i % len(sets)], cps[i % len(sets)]
        m.causal_conv1d_fwd(d["u"], c["weight"], c["bias"], c["init"],
                            out=u_bufs[i % len(sets)])

    def fused(i):
        d, c = sets[i % len(sets)], cps[i % len(sets)]
        m.selective_scan_fwd_conv(d["u"], c["weight"], d["delta"], d["A"], d["B"],
                                  d["C"], conv_bias=c["bias"], conv_init=c["init"],
                                  D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                                  softplus=s.softplus, last_state=d["last"],
                                  out=d["out"])

    def separate(i):
        conv(i)
        d = sets[i % len(sets)]
        m.selective_scan_fwd(u_bufs[i % len(sets)], d["delta"], d["A"], d["B"], d["C"],
                             D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                             softplus=s.softplus, last_state=d["last"], out=d["out"])

    conv_ms = _time(torch, stream, conv, steps)
    sep_ms = _time(torch, stream, separate, steps)
    pairs = [(hev.create(), hev.create()) for _ in range(steps)]
    k = [0]

    def fused_timed(i):
        if k[0] < len(pairs):
            m.set_scan_timing_events(*pairs[k[0]])
        k[0] += 1
        fused(i)
    for i in range(3):
        fused(i)
    torch.cuda.synchronize()
    k[0] = 0
    fused_ms = _time(torch, stream, fused_timed, steps, warmup=0)
    m.set_scan_timing_events(None, None)
    main_ms = sum(hev.elapsed_ms(a, b) for a, b in pairs) / steps
    for a, b in pairs:
        hev.destroy(a)
        hev.destroy(b)
    cb = W.conv_bytes(s)
    cgbs = cb / (conv_ms * 1e-3) / 1e9
    fused_bytes = W.scan_bytes(s) + 4 * s.dim * 5 + s.batch * s.dim * 3 * (2 if s.io == "bf16" else 4)
    slots = (s.state_elements * SLOTS_PER_STATE_ELEM +
             s.elements * (SLOTS_PER_ELEM + CONV_SLOTS_PER_ELEM))
    achieved = slots / (main_ms * 1e-3) / 1e12
    return {"workload": "causal conv width 4 + silu feeding the scan on %s" % s.name,
            "conv_ms": round(conv_ms, 5),
            "conv_roofline": {"bound": "hbm", "achieved": round(cgbs, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(cgbs / HBM_PEAK_GBS, 4), "traffic": None,
                              "kernel": "causal_conv1d_kernel",
                              "algorithmic_bytes": cb},
            "separate_conv_then_scan_ms": round(sep_ms, 5),
            "fused_ms": round(fused_ms, 5),
            "fused_speedup_vs_separate": round(sep_ms / fused_ms, 3),
            "fused_extra_ms_vs_scan_alone": round(fused_ms - scan_ms, 5),
            "fused_algorithmic_bytes": fused_bytes,
            "fused_gb_per_s": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1),
            "fused_roofline": {"bound": "alu", "achieved": round(achieved, 3),
                               "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                               "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
                               "traffic": None,
                               "kernel": "scan_kernel with the conv (main pass)",
                               "kernel_ms": round(main_ms, 5)}}


def bench_backward(torch, W, m, dev, s, sets, hev, steps, time_segments=0):
    """The backward of the same workload: gradients of every input for a
    seeded dout, rotating over the same input sets.  Reports the whole call
    (B/C pack, main kernel, group and batch sums) and the main kernel alone."""
    grads = [W.make_scan_grads(W.spec(s.name, seed=s.seed + 1000 * r, dstate=s.dstate))["dout"].to(dev)
             for r in range(len(sets))]

    def step(i):
        d = sets[i % len(sets)]
        return m.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"],
                                    grads[i % len(sets)], D=d["D"], z=d["z"],
                                    delta_bias=d["delta_bias"], softplus=s.softplus,
                                    time_segments=time_segments)
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    pairs = [(hev.create(), hev.create()) for _ in range(steps)]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        m.set_scan_timing_events(*pairs[i])
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    m.set_scan_timing_events(None, None)
    ms = e0.elapsed_time(e1) / steps
    main_ms = sum(hev.elapsed_ms(a, b) for a, b in pairs) / steps
    for a, b in pairs:
        hev.destroy(a)
        hev.destroy(b)
    nb = W.scan_bwd_bytes(s)
    slots = (s.state_elements * BWD_SLOTS_PER_STATE_ELEM +
             s.elements * BWD_SLOTS_PER_ELEM)
    achieved = slots / (main_ms * 1e-3) / 1e12
    return {"workload": "backward of %s: gradients of u, delta, z, A, B, C, D, "
                        "delta_bias for a seeded dout" % s.name,
            "steps": steps, "ms_per_step": round(ms, 5),
            "algorithmic_bytes": nb,
            "effective_gb_per_s": round(nb / (ms * 1e-3) / 1e9, 1),
            "gelem_per_s": round(s.state_elements / (ms * 1e-3) / 1e9, 2),
            "roofline": {"bound": "alu", "achieved": round(achieved, 3),
                         "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                         "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
                         "traffic": None,
                         "kernel": "bwd_pass_f + bwd_combine + bwd_pass_r",
                         "kernel_ms": round(main_ms, 5)}}


def software(torch):
    """Versions of the stack the numbers come from."""
    import numpy
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "numpy": numpy.__version__,
            "device": torch.cuda.get_device_properties(0).name}


def bench_decode(torch, W, m, dev, steps):
    """The decode workload: `steps` single-token updates of one in-place fp32
    state (84 MB, fits the 256 MB Infinity Cache, so the rate is an effective
    one), cycling through a ring of seeded tokens."""
    s = W.spec("decode", steps=steps)
    par = W.make_decode_params(s)
    toks = [{k: v.to(dev) for k, v in W.make_decode_token(s, k).items()}
            for k in range(s.tokens)]
    state = par["state"].to(dev)
    A, D, bias = par["A"].to(dev), par["D"].to(dev), par["dt_bias"].to(dev)
    out = torch.empty(s.batch, s.dim, dtype=torch.bfloat16, device=dev)

    def run(n):
        for i in range(n):
            t = toks[i % len(toks)]
            m.selective_state_update(state, t["x"], t["dt"], A, t["B"], t["C"], D=D,
                                     z=t["z"], dt_bias=bias, out=out)
    run(20)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nb = W.decode_step_bytes(s)
    # the same steps over 4 state buffers in turn (336 MB, more than the
    # 256 MB Infinity Cache holds): the rate from HBM
    states = [par["state"].to(dev) for _ in range(4)]

    def run_rot(n):
        for i in range(n):
            t = toks[i % len(toks)]
            m.selective_state_update(states[i % 4], t["x"], t["dt"], A, t["B"], t["C"],
                                     D=D, z=t["z"], dt_bias=bias, out=out)
    run_rot(8)
    torch.cuda.synchronize()
    e0.record()
    run_rot(steps)
    e1.record()
    torch.cuda.synchronize()
    ms_rot = e0.elapsed_time(e1) / steps
    return {"workload": "decode: %d sequences x D_inner %d, N %d, %d steps, bf16 tokens, "
                        "fp32 state in place" % (s.batch, s.dim, s.dstate, steps),
            "ms_per_step": round(ms, 5), "algorithmic_bytes_per_step": nb,
            "effective_gb_per_s": round(nb / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "rotating_4_states": {"ms_per_step": round(ms_rot, 5),
                                  "hbm_gb_per_s": round(nb / (ms_rot * 1e-3) / 1e9, 1),
                                  "pct_hbm_peak": round(100 * nb / (ms_rot * 1e-3) / 1e9 /
                                                        HBM_PEAK_GBS, 2)}}


def cpu_baseline(s, inp, seconds, nbytes):
    """The fp64 oracle on the host cores over the whole workload (all rows,
    all timesteps), repeated until about `seconds` of wall time, reported in
    the GPU value's unit."""
    import oracle
    nth = oracle.default_threads()
    conv = {k: oracle._f64(v) for k, v in inp.items() if k != "softplus"}
    reps, total = 0, 0.0
    while total < seconds:
        t0 = time.perf_counter()
        oracle.scan(conv["u"], conv["delta"], conv["A"], conv["B"], conv["C"],
                    D=conv["D"], z=conv["z"], delta_bias=conv["delta_bias"],
                    softplus=s.softplus, nthreads=nth)
        total += time.perf_counter() - t0
        reps += 1
    per = total / reps
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", "cores": nth,
            "kind": "oracle", "gelem_per_s": round(s.state_elements / per / 1e9, 3),
            "sample": "whole workload (%d rows x %d timesteps x N %d), %d run(s), "
                      "%.2f s each, fp64" % (s.batch * s.dim, s.seqlen, s.dstate, reps, per)}


def copy_calibration(torch):
    """torch's device copy of a 1 GiB buffer, 5 times: 1 GiB read + 1 GiB
    written per launch, the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def _counter_sum(d, kernel_substr, counter):
    """(sum over dispatches, number of dispatches) of a counter (summed over
    its instances) for the kernels whose name contains kernel_substr."""
    import sqlite3
    total, n = 0.0, 0
    for db in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
        c = sqlite3.connect(db)
        for (v,) in c.execute(
                "select sum(counter_value) from pmc_events where counter_name = ? and "
                "name like ? group by dispatch_id", (counter, "%" + kernel_substr + "%")):
            total += v
            n += 1
    if not n:
        raise RuntimeError("no %s samples for %s in %s" % (counter, kernel_substr, d))
    return total, n


def _counter_mean(d, kernel_substr, counter):
    total, n = _counter_sum(d, kernel_substr, counter)
    return total / n


# the kernels of one forward call (one B/C pack per call)
FWD_KERNELS = ("mssm::fwd::bc_pack_kernel", "mssm::fwd::scan_kernel<",
               "mssm::fwd::combine_kernel")


def _library_kernels(d, counter):
    """Names of the library's kernels with samples of a counter in a run."""
    import sqlite3
    names = set()
    for db in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
        c = sqlite3.connect(db)
        names.update(n for (n,) in c.execute(
            "select distinct name from pmc_events where counter_name = ?", (counter,))
            if "mssm::" in n)
    return names


def traffic_record(workload, time_segments, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes per forward call (all its kernels: the B/C pack, the scan
    launches on both streams and the segment combine) from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter reads
    for torch's copy of a 1 GiB buffer (1 GiB fetched, 1 GiB written)."""
    import workloads as W
    copy_kib = float(1 << 20)
    f_factor = copy_kib / _counter_mean(cfetch_dir, "copyBuffer", "FETCH_SIZE")
    w_factor = copy_kib / _counter_mean(cwrite_dir, "copyBuffer", "WRITE_SIZE")
    s = W.spec(workload)
    # the counter runs must hold this workload's forward calls only: another
    # forward scan (another state size) or another kernel of the library
    # would be counted as part of the call or change the call count
    scan_n = "mssm::fwd::scan_kernel<%d," % s.dstate
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        foreign = sorted(n for n in _library_kernels(d, counter)
                         if not any(k in n for k in FWD_KERNELS)
                         or ("fwd::scan_kernel<" in n and scan_n not in n))
        if foreign:
            raise RuntimeError("%s holds other kernels of the library (%s): profile the "
                               "forward of %s alone" % (d, foreign[0][:80], workload))
    _, calls = _counter_sum(fetch_dir, FWD_KERNELS[0], "FETCH_SIZE")
    fk = sum(_counter_sum(fetch_dir, k, "FETCH_SIZE")[0] for k in FWD_KERNELS) / calls
    wk = sum(_counter_sum(write_dir, k, "WRITE_SIZE")[0] for k in FWD_KERNELS) / calls
    import selective_state_space_52_amd as m
    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen, time_segments=time_segments)
    rec = {workload: {
        "kernel_source_sha256_16": kernel_source_hash(),
        "segments": plan["segments"],
        "calls": calls,
        "fetch_kib_per_call": round(fk, 1), "write_kib_per_call": round(wk, 1),
        "copy_fetch_factor": round(f_factor, 5), "copy_write_factor": round(w_factor, 5),
        "hbm_bytes_per_call": int(round((fk * f_factor + wk * w_factor) * 1024)),
        "algorithmic_bytes": W.scan_bytes(s)}}
    print(json.dumps(rec, indent=1))


def mamba2_traffic_record(fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes per Mamba-2 scan call (all its kernels: the scan launches
    and, when rows are cut in time, the combine) from FETCH_SIZE and
    WRITE_SIZE, scaled as for the forward scan by torch's 1 GiB copy."""
    import workloads as W
    copy_kib = float(1 << 20)
    f_factor = copy_kib / _counter_mean(cfetch_dir, "copyBuffer", "FETCH_SIZE")
    w_factor = copy_kib / _counter_mean(cwrite_dir, "copyBuffer", "WRITE_SIZE")
    try:   # one combine per call when the rows are cut in time
        _, calls = _counter_sum(fetch_dir, "mamba2_combine_kernel", "FETCH_SIZE")
    except RuntimeError:
        _, calls = _counter_sum(fetch_dir, "mamba2_scan_kernel", "FETCH_SIZE")
    fk, _ = _counter_sum(fetch_dir, "mamba2_", "FETCH_SIZE")
    wk, _ = _counter_sum(write_dir, "mamba2_", "WRITE_SIZE")
    s = W.spec("mamba2_2p7b_layer")
    rec = {"mamba2_2p7b_layer": {
        "kernel_source_sha256_16": kernel_source_hash(MAMBA2_SOURCES),
        "calls": calls,
        "fetch_kib_per_call": round(fk / calls, 1), "write_kib_per_call": round(wk / calls, 1),
        "copy_fetch_factor": round(f_factor, 5), "copy_write_factor": round(w_factor, 5),
        "hbm_bytes_per_call": int(round((fk * f_factor + wk * w_factor) / calls * 1024)),
        "algorithmic_bytes": W.mamba2_bytes(s)}}
    print(json.dumps(rec, indent=1))


def load_mamba2_traffic():
    """The recorded HBM bytes per Mamba-2 call, if taken with this kernel source."""
    try:
        with open(MAMBA2_TRAFFIC_FILE) as f:
            rec = json.load(f).get("mamba2_2p7b_layer")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash(MAMBA2_SOURCES):
        return None
    return rec.get("hbm_bytes_per_call")


def _kname(name: str) -> str:
    """Kernel name without its parameter list."""
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def rocprof_summary(d):
    """Per-kernel launch count and duration (and counter means) of a rocprofv3
    output directory, as text."""
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    for db in dbs:
        c = sqlite3.connect(db)
        print("# %s" % os.path.relpath(db, d))
        try:
            rows = c.execute("select name, stream_id, grid_x / workgroup_x, count(*), "
                             "avg(duration), min(duration), max(duration) from kernels "
                             "group by name, stream_id, grid_x / workgroup_x "
                             "order by sum(duration) desc").fetchall()
            print("%-62s %6s %6s %6s %10s %10s %10s" % ("kernel", "stream", "wgs", "calls",
                                                       "avg_us", "min_us", "max_us"))
            for name, st, wgs, n, avg, mn, mx in rows:
                print("%-62s %6s %6d %6d %10.2f %10.2f %10.2f" % (
                    _kname(name)[:62], st, wgs, n, avg / 1e3, mn / 1e3, mx / 1e3))
        except sqlite3.Error:
            pass
        try:
            # one line per kernel, stream and grid: launches of one kernel
            # with different roles (a main pass, an aggregate pass) apart
            rows = c.execute(
                "select p.name, k.stream_id, k.grid_x / k.workgroup_x, p.counter_name, "
                "count(*), avg(p.v), avg(k.duration) from (select name, dispatch_id, "
                "counter_name, sum(counter_value) as v from pmc_events group by name, "
                "dispatch_id, counter_name) p join kernels k on k.dispatch_id = "
                "p.dispatch_id group by p.name, k.stream_id, k.grid_x / k.workgroup_x, "
                "p.counter_name order by p.name, k.stream_id, 3, p.counter_name").fetchall()
            if rows:
                print("%-62s %6s %6s %-24s %6s %16s %10s" % (
                    "kernel", "stream", "wgs", "counter", "n", "mean/dispatch", "avg_us"))
            for name, st, wgs, cn, n, v, dur in rows:
                print("%-62s %6s %6d %-24s %6d %16.1f %10.2f" % (
                    _kname(name)[:62], st, wgs, cn, n, v, dur / 1e3))
        except sqlite3.Error:
            pass


if __name__ == "__main__":
    main()
