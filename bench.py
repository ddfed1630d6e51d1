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
CUS, CLOCK_GHZ = 256, 2.4
# fp32 VALU issue peak: 128 lanes per CU per clock (MI355X's 157.3 TFLOP/s fp32
# vector peak counts one fma as 2 flops).  Plain, unpacked v_fma_f32 reaches
# it only with several waves ready per SIMD: the library's probe measured 44,
# 83, 93 and 99 fma lanes per CU per clock at 1, 2, 4 and 8 waves per SIMD
# (bench.py --alu-probe).
VALU_LANES_PER_CU_CLK = 128
VALU_PEAK_TSLOTS = CUS * VALU_LANES_PER_CU_CLK * CLOCK_GHZ / 1e3   # 78.64 T lane-slots/s
# Transcendentals (v_exp_f32, v_log_f32, v_rcp_f32) issue at a quarter of that
# (the probe: 30 exp lanes per CU per clock at 8 waves per SIMD)
EXP_PEAK_T = VALU_PEAK_TSLOTS / 4                          # 19.66 T exp/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_main_traffic.json")
# the sources the forward scan kernel is built from (the traffic record is
# tied to them)
KERNEL_SOURCES = [os.path.join(ROOT, "selective_state_space_52_amd", "csrc", f)
                  for f in ("scan_fwd_impl.h", "scan_fwd.hip", "scan_fwd_n16.hip",
                            "scan_common.h", "dev_math.h")]

# Algorithmic VALU issue slots of the scan (fp32, one lane = one slot; a
# transcendental occupies four slots, as v_exp/v_log/v_rcp issue at a quarter
# of the fma rate).  Per state element: Delta*A (1), exp (4), Delta*u times B
# (1), the state fma (1), the C readout fma (1).  Per element: delta + bias
# (1), softplus = exp + log1p (4 + 4 + 3), Delta*u (1), D skip fma (1),
# silu = exp + reciprocal (4 + 4 + 2), gate multiply (1), bf16 rounding (1).
SLOTS_PER_STATE_ELEM = 8
SLOTS_PER_ELEM = 26
# The backward, counted the same way for the algorithm itself (one forward
# sweep keeping h_t, one reverse sweep), not for the kernel's recompute.  Per
# state element: the forward recurrence (7) and the C readout for dz (1); in
# reverse g += dy C, dy h (dC term), g Delta u (dB term), sum g B, g e, (g e)
# h_prev, sum A (g e h_prev), dA accumulate (8); one add each for the
# channel sums of dB and dC (2).  Per element: delta + bias (1), softplus
# (13), sigmoid of delta + bias (10), Delta*u (1), sigmoid of z (10),
# dy = dout z sigmoid(z) (2), dout silu'(z) (4), du (2), dDelta (1), ddelta
# (1), dz (2), dD and dbias accumulates (2).
BWD_SLOTS_PER_STATE_ELEM = 18
BWD_SLOTS_PER_ELEM = 49
# The width-4 causal conv in the fused path adds per element: 4 fmas and
# silu = exp + reciprocal (4 + 4) + 3, i.e. 15 slots.
CONV_SLOTS_PER_ELEM = 15


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
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other forward workloads and the 1-thread oracle runs")
    ap.add_argument("--only-forward", action="store_true",
                    help="time the workload's forward calls alone (profiling runs)")
    ap.add_argument("--backward-steps", type=int, default=20)
    ap.add_argument("--bwd-time-segments", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-mamba2", action="store_true")
    ap.add_argument("--only-mamba2", action="store_true",
                    help="run the Mamba-2 scan leg alone (profiling runs)")
    ap.add_argument("--mamba2-traffic-record", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    ap.add_argument("--mamba2-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--alu-probe", action="store_true",
                    help="only the ALU issue-rate probes and the ceiling they give")
    ap.add_argument("--rocprof-summary", default=None)
    ap.add_argument("--call-breakdown", default=None, metavar="KERNEL_TRACE_DIR",
                    help="per-call timeline of the 2.8B-shaped forward calls in a "
                         "rocprofv3 kernel trace (B/C pack, gap, scan launch)")
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


def load_traffic(workload: str, plan: dict, key: str = "main_pass_hbm_bytes_per_launch"):
    """HBM bytes from the committed counter record of this workload's forward:
    per launch of the scan kernel (the kernel the roofline is about; one per
    call), or per call (the B/C pack and the scan launch).  None when the
    record is missing or was taken on another version of the kernel source."""
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
    return rec.get(key)


def hbm_roofline(nbytes: float, ms: float, kernel: str, kernel_ms: float, traffic=None):
    """HBM roofline entry: algorithmic bytes of one launch over its duration."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
            "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes_per_launch": int(nbytes)}


def alu_figures(slots: float, ms: float, nbytes: float):
    """Algorithmic VALU issue slots against the chip's issue peak, and the HBM
    fraction those slots allow at 100% issue (the path's ALU ceiling)."""
    t_alu = slots / (VALU_PEAK_TSLOTS * 1e12)                 # s at full issue
    ceiling = nbytes / t_alu / 1e9 / HBM_PEAK_GBS
    achieved = slots / (ms * 1e-3) / 1e12
    return {"achieved": round(achieved, 3), "peak": round(VALU_PEAK_TSLOTS, 3),
            "unit": "Tslot/s", "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
            "slots_per_element": None, "ceiling_frac_of_hbm_peak": round(ceiling, 4)}


def scan_slots(s) -> float:
    return s.state_elements * SLOTS_PER_STATE_ELEM + s.elements * SLOTS_PER_ELEM


def make_sets(torch, W, dev, name, rotate, **over):
    s = W.spec(name, **over)
    sets = []
    for r in range(max(1, rotate)):
        inp = W.make_scan_inputs(s if r == 0 else W.spec(name, seed=s.seed + 1000 * r, **over))
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        d["out"] = torch.empty_like(d["u"])
        d["last"] = torch.empty(s.batch, s.dim, s.dstate, device=dev)
        sets.append(d)
    return s, sets


def scan_leg(torch, W, m, dev, hev, s, sets, steps, warmup, time_segments=0):
    """One forward workload: W untimed calls, then exactly `steps` timed calls
    (events on the caller's stream around them, synchronised on both sides),
    then the same calls again with HIP events around the scan kernel (the
    call's one launch after the B/C pack) for its own duration."""
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i % len(sets)]
        m.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], D=d["D"],
                             z=d["z"], delta_bias=d["delta_bias"],
                             softplus=s.softplus, last_state=d["last"],
                             out=d["out"], time_segments=time_segments)
    settle_gpu(torch, dev)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    pairs = [(hev.create(), hev.create()) for _ in range(steps)]
    for i in range(steps):
        m.set_scan_timing_events(*pairs[i])
        step(i)
    torch.cuda.synchronize()
    m.set_scan_timing_events(None, None)
    per = sorted(hev.elapsed_ms(a, b) for a, b in pairs)
    for a, b in pairs:
        hev.destroy(a)
        hev.destroy(b)
    io = torch.bfloat16 if s.io == "bf16" else torch.float32
    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen, io, time_segments)
    nbytes = W.scan_bytes(s)
    kernel_ms = sum(per) / len(per)
    # the timed kernel is the call's one scan launch (every task of the call;
    # only the B/C pack runs before it)
    share = 1.0
    slots = scan_slots(s)
    alu = alu_figures(slots * share, kernel_ms, nbytes * share)
    alu["slots_per_element"] = round(slots / s.elements, 2)
    return {"ms": ms, "wall_s": wall, "kernel_ms": kernel_ms,
            "kernel_ms_median": per[len(per) // 2], "kernel_ms_min": per[0],
            "plan": plan, "bytes": nbytes, "share": share, "alu": alu,
            "alu_call": alu_figures(slots, ms, nbytes)}


def config_entry(s, W, r, ms_key="ms"):
    """Extra-key summary of one forward workload."""
    ms = r[ms_key]
    gbs = r["bytes"] / (ms * 1e-3) / 1e9
    return {"workload": "%s: batch %d, D_inner %d, N %d, L %d, %s" % (
                s.name, s.batch, s.dim, s.dstate, s.seqlen, s.io),
            "ms_per_call": round(ms, 5), "gb_per_s": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "gelem_per_s": round(s.state_elements / (ms * 1e-3) / 1e9, 2),
            "alu_frac": r["alu_call"]["frac"],
            "alu_ceiling_frac_of_hbm_peak": r["alu_call"]["ceiling_frac_of_hbm_peak"],
            "main_kernel_ms": round(r["kernel_ms"], 5), "plan": r["plan"],
            "algorithmic_bytes": r["bytes"]}


def main():
    args = parse()
    if args.rocprof_summary:
        rocprof_summary(args.rocprof_summary)
        return
    if args.call_breakdown:
        call_breakdown(args.call_breakdown)
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hev = HipEvents()
    if args.only_mamba2:
        print(json.dumps({"mamba2": bench_mamba2(torch, W, m, dev, args.mamba2_steps)}),
              flush=True)
        return
    if args.alu_probe:
        s = W.spec(args.workload)
        print(json.dumps({"alu_probe": alu_probe(torch, m, dev, s, W.scan_bytes(s),
                                                 sweep=(4, 8, 16, 32))}),
              flush=True)
        return
    if args.only_forward:
        # profiling runs: the headline workload's forward calls alone
        over = {"dstate": args.dstate} if args.dstate else {}
        s, sets = make_sets(torch, W, dev, args.workload, args.rotate, **over)
        r = scan_leg(torch, W, m, dev, hev, s, sets, args.steps, args.warmup,
                     args.time_segments)
        print(json.dumps(config_entry(s, W, r)), flush=True)
        return

    over = {"dstate": args.dstate} if args.dstate else {}
    s, sets = make_sets(torch, W, dev, args.workload, args.rotate, **over)
    extra = {}
    # The other legs run first: the headline is then timed on a GPU whose
    # clocks have left their idle state (the first ~100 calls of a fresh
    # process run ~10% slower).
    if not args.no_decode:
        extra["decode"] = bench_decode(torch, W, m, dev, args.decode_steps)
    if not args.no_backward and s.dstate <= 32:   # the backward takes N <= 32
        extra["backward"] = bench_backward(torch, W, m, dev, s, sets, hev,
                                           args.backward_steps, args.bwd_time_segments)
    if not args.no_conv:
        extra["conv"] = bench_conv(torch, W, m, dev, s, sets, hev)
    if not args.no_mamba2:
        extra["mamba2"] = bench_mamba2(torch, W, m, dev, args.mamba2_steps)
    if not args.no_configs:
        extra["configs"] = bench_other_configs(torch, W, m, dev, hev, args)

    r = scan_leg(torch, W, m, dev, hev, s, sets, args.steps, args.warmup, args.time_segments)
    clock = shader_clock_mhz()
    ms = r["ms"]
    nbytes = r["bytes"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    plan = r["plan"]
    traffic = load_traffic(args.workload, plan)
    traffic_call = load_traffic(args.workload, plan, "hbm_bytes_per_call")
    roof = hbm_roofline(nbytes * r["share"], r["kernel_ms"],
                        "scan_kernel: the call's one scan launch (%d whole channel groups, "
                        "%d groups cut into %d time segments with their aggregates)" % (
                            plan["whole_groups"], plan["split_groups"], plan["segments"]),
                        r["kernel_ms"], traffic)
    roof["kernel_ms_median"] = round(r["kernel_ms_median"], 5)
    roof["kernel_ms_min"] = round(r["kernel_ms_min"], 5)
    roof["alu"] = r["alu"]
    roof["binding_resource"] = "valu"
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
        "gelem_per_s": round(s.state_elements / (ms * 1e-3) / 1e9, 2),
        "roofline": roof,
        "alu_call": r["alu_call"],
        "call_minus_kernel_ms": round(ms - r["kernel_ms"], 5),
        "exp_rate": {"achieved": round(s.state_elements * r["share"] /
                                       (r["kernel_ms"] * 1e-3) / 1e12, 3),
                     "peak": round(EXP_PEAK_T, 3), "unit": "T exp/s"},
        "wall_s": round(r["wall_s"], 3),
        "software": software(torch),
        "copy_ceiling": copy_ceiling(torch, dev),
        "shader_clock_mhz": clock,
    }
    res["alu_probe"] = alu_probe(torch, m, dev, s, nbytes * r["share"], r["kernel_ms"])
    res["roofline"]["traffic_per_call"] = traffic_call
    res["roofline"]["frac_of_copy_ceiling"] = round(
        roof["achieved"] / res["copy_ceiling"]["gb_per_s"], 4)
    res.update(extra)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(W, s, sets, args.cpu_seconds, nbytes)
        if not args.no_configs:
            res["cpu_baseline"]["single_thread"] = cpu_single_thread(W)
    print(json.dumps(res), flush=True)


def probe_rates(torch, m, dev, waves_per_cu, iters=4096, reps=10):
    """Measured issue rates (per second) of the library's ALU probe kernels
    at `waves_per_cu` resident waves per CU: fp32 fma (kind 0), v_exp_f32
    (kind 1), state elements of the scan's inner-step mix (kind 2) and state
    elements of the same recurrence as an in-wave associative scan over 64
    timesteps (kind 3), and iterations of 8 fma plus 2 exp on independent
    chains (kind 4)."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = cus * waves_per_cu // 4        # 256-thread workgroups: 4 waves
    threads = blocks * 256
    sink = torch.empty(threads, device=dev)
    rates = {}
    for kind, per_iter in ((0, 8), (1, 8), (2, 4), (3, 4), (4, 1)):
        for _ in range(2):
            m.valu_probe(kind, blocks, iters, sink)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            m.valu_probe(kind, blocks, iters, sink)
        b.record()
        torch.cuda.synchronize()
        rates[kind] = per_iter * iters * threads * reps / (a.elapsed_time(b) * 1e-3)
    return rates


def alu_probe(torch, m, dev, s=None, nbytes=None, kernel_ms=None, sweep=(16, 32)):
    """Issue rates of the vector ALU measured on this GPU with the library's
    probe kernels (mssm_valu_probe): fp32 fma alone, v_exp_f32 alone, and the
    scan's state-element mix (a multiply, an exponential, a multiply, the state
    fma and the readout fma per state element), at each occupancy in `sweep`
    (waves per CU; the forward scan runs 16: two 8-wave workgroups).  From the
    rates at the scan's occupancy, its ALU ceiling for workload `s`: the state
    elements at the measured mix rate plus the per-element work
    (SLOTS_PER_ELEM fma slots) at the measured fma rate, and the fraction of
    that ceiling the scan kernel reaches."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    settle_gpu(torch, dev)
    res = {"launch": "CUs x waves/4 workgroups of 256 threads, 4096 iterations",
           "by_waves_per_cu": {}}
    at = {}
    for w in sweep:
        r = probe_rates(torch, m, dev, w)
        at[w] = r
        res["by_waves_per_cu"][str(w)] = {
            "fma_T_per_s": round(r[0] / 1e12, 3), "exp_T_per_s": round(r[1] / 1e12, 3),
            "state_element_mix_T_per_s": round(r[2] / 1e12, 3),
            "fma_slots_per_state_element": round(r[0] / r[2], 3),
            "wave_scan_state_elements_T_per_s": round(r[3] / 1e12, 3),
            # 8 fma + 2 exp on independent chains: time per iteration against
            # the two kinds' own times added (1: no overlap) and against the
            # longer of the two (the fraction of the shorter one hidden)
            "fma_exp_mix_time_vs_sum": round((1 / r[4]) / (8 / r[0] + 2 / r[1]), 3),
            "fma_exp_overlap_frac": round(((8 / r[0] + 2 / r[1]) - 1 / r[4]) /
                                          min(8 / r[0], 2 / r[1]), 3)}
    clock = shader_clock_mhz()
    res["shader_clock_mhz"] = clock
    if clock:
        for w, r in at.items():
            per_clk = 1.0 / (cus * clock * 1e6)
            res["by_waves_per_cu"][str(w)]["per_cu_per_clock"] = {
                "fma": round(r[0] * per_clk, 2), "exp": round(r[1] * per_clk, 2),
                "state_elements": round(r[2] * per_clk, 2),
                "wave_scan_state_elements": round(r[3] * per_clk, 2)}
    if s is not None:
        r = at[16] if 16 in at else at[max(at)]
        ceil_s = s.state_elements / r[2] + s.elements * SLOTS_PER_ELEM / r[0]
        res["scan_ceiling_ms"] = round(ceil_s * 1e3, 5)
        res["scan_ceiling_frac_of_hbm_peak"] = round(nbytes / ceil_s / 1e9 / HBM_PEAK_GBS, 4)
        if kernel_ms:
            res["scan_kernel_frac_of_ceiling"] = round(ceil_s * 1e3 / kernel_ms, 4)
    return res


def bench_other_configs(torch, W, m, dev, hev, args):
    """The other forward workloads, each timed as the headline is: the tiny
    fp32 case, the 130M-shaped layer and the long sequence in one call and as
    64 chained calls of 2048 steps carrying last_state."""
    out = {}
    for name, rot, steps in (("tiny_f32", 1, 50), ("mamba130m_layer", 3, 50),
                             ("long_chunked", 1, 5)):
        s, sets = make_sets(torch, W, dev, name, rot)
        r = scan_leg(torch, W, m, dev, hev, s, sets, steps, 3)
        e = config_entry(s, W, r)
        if name == "long_chunked":
            d = sets[0]
            stream = torch.cuda.current_stream(dev)
            pieces = [(a, min(s.seqlen, a + s.chunk)) for a in range(0, s.seqlen, s.chunk)]
            parts = [{k: (d[k][..., a:b].contiguous() if k in ("u", "delta", "z") else
                          d[k][:, a:b].contiguous() if k in ("B", "C") else d[k])
                      for k in ("u", "delta", "z", "B", "C")} for a, b in pieces]
            outs = [torch.empty_like(p["u"]) for p in parts]
            state = torch.zeros(s.batch, s.dim, s.dstate, device=dev)

            def chained(_):
                state.zero_()
                for p, o in zip(parts, outs):
                    m.selective_scan_fwd(p["u"], p["delta"], d["A"], p["B"], p["C"], D=d["D"],
                                         z=p["z"], delta_bias=d["delta_bias"],
                                         softplus=s.softplus, last_state=state,
                                         load_state=True, out=o)
            settle_gpu(torch, dev)
            cms = _time(torch, stream, chained, 3, warmup=1)
            e["chained_2048_step_calls_ms"] = round(cms, 5)
            e["chained_hbm_frac"] = round(r["bytes"] / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            del parts, outs
        out[name] = e
        del sets
        torch.cuda.empty_cache()
    return out


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
    settle_gpu(torch, dev)
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


def bench_conv(torch, W, m, dev, s, sets, hev, steps=20):
    """The causal conv (width 4, silu) ahead of the scan on the same workload:
    the standalone conv kernel (HBM-bound), its backward (dx, dweight, dbias
    for a dout of the same shape), and the conv fused into the scan's load
    stage, against running the two one after the other."""
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

    def scan_alone(i):
        d = sets[i % len(sets)]
        m.selective_scan_fwd(d["u"], d["delta"], d["A"], d["B"], d["C"],
                             D=d["D"], z=d["z"], delta_bias=d["delta_bias"],
                             softplus=s.softplus, last_state=d["last"], out=d["out"])

    def conv_bwd(i):
        d, c = sets[i % len(sets)], cps[i % len(sets)]
        m.causal_conv1d_bwd(d["u"], c["weight"], d["z"], bias=c["bias"], init=c["init"])

    settle_gpu(torch, dev)
    conv_ms = _time(torch, stream, conv, steps)
    conv_bwd_ms = _time(torch, stream, conv_bwd, steps)
    sep_ms = _time(torch, stream, separate, steps)
    scan_ms = _time(torch, stream, scan_alone, steps)
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
            "conv_bwd_ms": round(conv_bwd_ms, 5),
            "conv_bwd_roofline": {"bound": "hbm",
                                  "achieved": round(W.conv_bwd_bytes(s) / (conv_bwd_ms * 1e-3)
                                                    / 1e9, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(W.conv_bwd_bytes(s) / (conv_bwd_ms * 1e-3) /
                                                1e9 / HBM_PEAK_GBS, 4),
                                  "traffic": None, "kernel": "causal_conv1d_bwd_kernel",
                                  "algorithmic_bytes": W.conv_bwd_bytes(s)},
            "separate_conv_then_scan_ms": round(sep_ms, 5),
            "fused_ms": round(fused_ms, 5),
            "fused_speedup_vs_separate": round(sep_ms / fused_ms, 3),
            "scan_alone_ms": round(scan_ms, 5),
            "fused_extra_ms_vs_scan_alone": round(fused_ms - scan_ms, 5),
            "fused_algorithmic_bytes": fused_bytes,
            "fused_gb_per_s": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1),
            "fused_roofline": {"bound": "hbm",
                               "achieved": round(fused_bytes / (fused_ms * 1e-3) / 1e9, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(fused_bytes / (fused_ms * 1e-3) / 1e9 /
                                             HBM_PEAK_GBS, 4),
                               "traffic": None,
                               "kernel": "scan_kernel with the conv (main pass)",
                               "kernel_ms": round(main_ms, 5),
                               "alu": {"achieved": round(achieved, 3),
                                       "peak": round(VALU_PEAK_TSLOTS, 3),
                                       "unit": "Tslot/s",
                                       "frac": round(achieved / VALU_PEAK_TSLOTS, 4)}}}


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
    settle_gpu(torch, dev)
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
            "roofline": {"bound": "hbm",
                         "achieved": round(nb / (ms * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": None,
                         "kernel": "whole backward call",
                         "passes_ms": round(main_ms, 5),
                         "alu": {"achieved": round(achieved, 3),
                                 "peak": round(VALU_PEAK_TSLOTS, 3), "unit": "Tslot/s",
                                 "frac": round(achieved / VALU_PEAK_TSLOTS, 4),
                                 "kernels": "bwd_pass_f + bwd_combine + bwd_pass_r"}}}


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
    settle_gpu(torch, dev)
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

    def run_rot(n, stream=False):
        for i in range(n):
            t = toks[i % len(toks)]
            m.selective_state_update(states[i % 4], t["x"], t["dt"], A, t["B"], t["C"],
                                     D=D, z=t["z"], dt_bias=bias, out=out, stream_state=stream)
    run_rot(8)
    torch.cuda.synchronize()
    e0.record()
    run_rot(steps)
    e1.record()
    torch.cuda.synchronize()
    ms_rot = e0.elapsed_time(e1) / steps
    # the same with the state streamed (non-temporal loads and stores, the
    # caller's hint for states that do not stay in the caches between steps)
    run_rot(8, True)
    torch.cuda.synchronize()
    e0.record()
    run_rot(steps, True)
    e1.record()
    torch.cuda.synchronize()
    ms_rot_nt = e0.elapsed_time(e1) / steps
    # The same rotating loop as one captured HIP graph of 64 steps, replayed:
    # the host enqueues one graph launch per 64 steps instead of 64 calls.
    G = 64
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_rot(G)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // G)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / (reps * G)
    del graph
    return {"workload": "decode: %d sequences x D_inner %d, N %d, %d steps, bf16 tokens, "
                        "fp32 state in place" % (s.batch, s.dim, s.dstate, steps),
            "ms_per_step": round(ms, 5), "algorithmic_bytes_per_step": nb,
            "effective_gb_per_s": round(nb / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "rotating_4_states": {"ms_per_step": round(ms_rot, 5),
                                  "hbm_gb_per_s": round(nb / (ms_rot * 1e-3) / 1e9, 1),
                                  "pct_hbm_peak": round(100 * nb / (ms_rot * 1e-3) / 1e9 /
                                                        HBM_PEAK_GBS, 2)},
            "rotating_4_states_stream_hint": {
                "ms_per_step": round(ms_rot_nt, 5),
                "hbm_gb_per_s": round(nb / (ms_rot_nt * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * nb / (ms_rot_nt * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)},
            "rotating_4_states_graph": {
                "ms_per_step": round(ms_graph, 5), "steps_per_graph": G,
                "hbm_gb_per_s": round(nb / (ms_graph * 1e-3) / 1e9, 1),
                "pct_hbm_peak": round(100 * nb / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}}


def cpu_baseline(W, s, sets, seconds, nbytes):
    """The fp64 oracle on the host cores over the whole workload (all rows,
    all timesteps, the first input set), repeated until about `seconds` of
    wall time, reported in the GPU value's unit."""
    import oracle
    nth = oracle.default_threads()
    d = sets[0]
    conv = {k: oracle._f64(d[k].cpu()) for k in ("u", "delta", "A", "B", "C", "D", "z",
                                                  "delta_bias")}
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
                      "%.2f s each, fp64, %d threads" % (s.batch * s.dim, s.seqlen, s.dstate,
                                                         reps, per, nth)}


def cpu_single_thread(W):
    """The oracle on one host thread, one run over each of the tiny, 130M- and
    2.8B-shaped workloads."""
    import oracle
    out = {}
    for name in ("tiny_f32", "mamba130m_layer", "mamba2p8b_layer"):
        s = W.spec(name)
        inp = W.make_scan_inputs(s)
        c = {k: oracle._f64(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z",
                                               "delta_bias")}
        t0 = time.perf_counter()
        oracle.scan(c["u"], c["delta"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"],
                    delta_bias=c["delta_bias"], softplus=s.softplus, nthreads=1)
        dt = time.perf_counter() - t0
        out[name] = {"s": round(dt, 3), "gb_per_s": round(W.scan_bytes(s) / dt / 1e9, 4),
                     "gelem_per_s": round(s.state_elements / dt / 1e9, 4)}
    return out


_COPY = {}


def settle_gpu(torch, dev, seconds=0.6):
    """Keep the GPU busy with device copies of 1 GiB for about `seconds`, and
    time the last of them: the HBM rate a plain streaming kernel reaches here
    (1 GiB read + 1 GiB written per copy).  A GPU that has idled (the host
    drawing inputs) runs the scan ~10% slower for its first few hundred
    milliseconds of work, so every timed leg starts right after this."""
    n = 1 << 30
    if "a" not in _COPY:
        _COPY["a"] = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        _COPY["b"] = torch.empty_like(_COPY["a"])
    a, b = _COPY["a"], _COPY["b"]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            b.copy_(a)
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ms = _time(torch, stream, lambda i: b.copy_(a), 20, warmup=0)
    _COPY["last"] = {"gb_per_s": round(2 * n / (ms * 1e-3) / 1e9, 1), "ms": round(ms, 4),
                     "kernel": "torch copy_ of 1 GiB"}
    return _COPY["last"]


def copy_ceiling(torch, dev):
    """The copy rate measured by the last settle_gpu (the plain streaming
    kernel's HBM rate on this GPU)."""
    return _COPY.get("last") or settle_gpu(torch, dev)


def shader_clock_mhz():
    """The shader clock level the amdgpu kernel module reports as current (sysfs
    pp_dpm_sclk), read right after the headline timing, or None."""
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        tok = line.split(":", 1)[1].strip().split()[0].lower()
                        return int(float(tok.replace("mhz", "")))
        except (OSError, ValueError, IndexError):
            continue
    return None


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


# the kernels of one forward call (one B/C pack per call, then one scan launch)
FWD_KERNELS = ("mssm::fwd::bc_pack", "mssm::fwd::scan_kernel<")


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


def _dispatches(d, counter):
    """(dispatch_id, kernel name, stream_id, workgroups, counter value summed
    over its instances) of every dispatch in a counter run, in dispatch order."""
    import sqlite3
    rows = []
    for db in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
        c = sqlite3.connect(db)
        rows += c.execute(
            "select p.dispatch_id, p.name, k.stream_id, k.grid_x / k.workgroup_x, "
            "sum(p.counter_value) from pmc_events p join kernels k on "
            "k.dispatch_id = p.dispatch_id where p.counter_name = ? "
            "group by p.dispatch_id order by p.dispatch_id", (counter,)).fetchall()
    if not rows:
        raise RuntimeError("no %s samples in %s" % (counter, d))
    return rows


def traffic_record(workload, time_segments, fetch_dir, write_dir, cfetch_dir, cwrite_dir):
    """HBM bytes of the forward from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for torch's copy of
    a 1 GiB buffer (1 GiB fetched, 1 GiB written): per launch of the scan
    kernel (one per call, every task of the call), and per call (the B/C pack
    and the scan launch)."""
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
    import selective_state_space_52_amd as m
    plan = m.scan_plan(s.batch, s.dim, s.dstate, s.seqlen, time_segments=time_segments)
    per = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = _dispatches(d, counter)
        lib = [r for r in rows if "mssm::" in r[1]]
        packs = [r for r in lib if FWD_KERNELS[0] in r[1]]
        mains = [r for r in lib if FWD_KERNELS[1] in r[1]]
        per[counter] = {"calls": len(packs),
                        "call_kib": sum(r[4] for r in lib) / len(packs),
                        "main_kib": sum(r[4] for r in mains) / max(1, len(mains)),
                        "main_launches": len(mains)}
    fk, wk = per["FETCH_SIZE"], per["WRITE_SIZE"]
    rec = {workload: {
        "kernel_source_sha256_16": kernel_source_hash(),
        "segments": plan["segments"],
        "calls": fk["calls"], "main_pass_launches": fk["main_launches"],
        "fetch_kib_per_call": round(fk["call_kib"], 1),
        "write_kib_per_call": round(wk["call_kib"], 1),
        "main_pass_fetch_kib_per_launch": round(fk["main_kib"], 1),
        "main_pass_write_kib_per_launch": round(wk["main_kib"], 1),
        "copy_fetch_factor": round(f_factor, 5), "copy_write_factor": round(w_factor, 5),
        "hbm_bytes_per_call": int(round((fk["call_kib"] * f_factor +
                                         wk["call_kib"] * w_factor) * 1024)),
        "main_pass_hbm_bytes_per_launch": int(round((fk["main_kib"] * f_factor +
                                                     wk["main_kib"] * w_factor) * 1024)),
        "algorithmic_bytes": W.scan_bytes(s),
        "main_pass_algorithmic_bytes": W.scan_bytes(s)}}
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


def call_breakdown(d, scan_prefix="mssm::fwd::scan_kernel<16, 8, true, "):
    """Per-call timeline of back-to-back forward calls of one workload in a
    rocprofv3 kernel trace: each B/C pack followed directly by that call's
    scan launch on the same stream.  Prints the pack's duration, the gap from
    the pack's end to the scan's start, the scan's duration, and the gap from
    the scan's end to the next call's pack (the host keeps the queue fed when
    that gap is a launch latency), in microseconds."""
    import sqlite3
    rows = []
    for db in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
        c = sqlite3.connect(db)
        rows += c.execute("select name, start, end, stream_id from kernels "
                          "order by start").fetchall()
    calls = []
    for i in range(len(rows) - 1):
        a, b = rows[i], rows[i + 1]
        if "fwd::bc_pack" in a[0] and _kname(b[0]).startswith(scan_prefix) and a[3] == b[3]:
            calls.append((a, b))
    if not calls:
        raise RuntimeError("no pack + scan pairs of %s in %s" % (scan_prefix, d))
    pack = [(a[2] - a[1]) / 1e3 for a, b in calls]
    gap = [(b[1] - a[2]) / 1e3 for a, b in calls]
    scan = [(b[2] - b[1]) / 1e3 for a, b in calls]
    # gaps to the next call's pack, for calls followed directly by another
    nxt = []
    for (a, b), (a2, _) in zip(calls, calls[1:]):
        if a2[1] > b[2]:
            nxt.append((a2[1] - b[2]) / 1e3)
    med = lambda v: sorted(v)[len(v) // 2]
    print("calls %d" % len(calls))
    for lab, v in (("pack_us", pack), ("pack_to_scan_gap_us", gap), ("scan_us", scan),
                   ("scan_to_next_pack_gap_us", nxt)):
        if v:
            print("%-26s median %8.2f  min %8.2f  max %8.2f" % (lab, med(v), min(v), max(v)))


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
