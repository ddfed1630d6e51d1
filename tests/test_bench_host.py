"""Host logic of bench.py on the CPU: the HBM traffic record built from
rocprofv3 counter databases (scaled by the copy calibration), its tie to the
kernel source, the roofline arithmetic, the per-call timeline of a kernel
trace, and the refusal of more than one GPU.  The counter databases here are
small SQLite files with the columns the bench reads, filled with known values."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PACK = "void mssm::fwd::bc_pack_tokens_kernel<2>(unsigned int const*)"
SCAN = ("void mssm::fwd::scan_kernel<16, 8, true, 3, true, true, false, false>"
        "(void const*)")
COPY = "__amd_rocclr_copyBuffer"


def write_db(d, name, dispatches, counter):
    """dispatches: (kernel name, [counter value per instance], start, end)."""
    os.makedirs(d, exist_ok=True)
    c = sqlite3.connect(os.path.join(d, name + "_results.db"))
    c.execute("create table kernels (dispatch_id, name, stream_id, grid_x, workgroup_x, "
              "duration, start, end)")
    c.execute("create table pmc_events (dispatch_id, name, counter_name, counter_value)")
    for i, (kname, vals, start, end) in enumerate(dispatches):
        c.execute("insert into kernels values (?,?,?,?,?,?,?,?)",
                  (i, kname, 0, 256 * 256, 256, end - start, start, end))
        for v in vals:
            c.execute("insert into pmc_events values (?,?,?,?)", (i, kname, counter, v))
    c.commit()
    c.close()


def forward_run(calls, pack_kib, scan_kib):
    """calls x (pack, scan) dispatches after one 1 GiB copy; each value split
    over two counter instances."""
    rows = [(COPY, [1.0, 2.0], 0, 100)]
    t = 1000
    for _ in range(calls):
        rows.append((PACK, [pack_kib / 2, pack_kib / 2], t, t + 3000))
        rows.append((SCAN, [scan_kib / 4, 3 * scan_kib / 4], t + 3000, t + 200000))
        t += 210000
    return rows


def test_traffic_record_scales_by_the_copy_counters(tmp_path, capsys):
    # the copy of 1 GiB reads as 512 MiB on FETCH_SIZE (factor 2) and 1 GiB on
    # WRITE_SIZE (factor 1)
    write_db(str(tmp_path / "cfetch"), "cfetch", [(COPY, [524288.0], 0, 1)] * 3, "FETCH_SIZE")
    write_db(str(tmp_path / "cwrite"), "cwrite", [(COPY, [1048576.0], 0, 1)] * 3, "WRITE_SIZE")
    write_db(str(tmp_path / "fetch"), "fetch", forward_run(4, 100.0, 1000.0), "FETCH_SIZE")
    write_db(str(tmp_path / "write"), "write", forward_run(4, 50.0, 500.0), "WRITE_SIZE")
    bench.traffic_record("mamba2p8b_layer", 0, str(tmp_path / "fetch"),
                         str(tmp_path / "write"), str(tmp_path / "cfetch"),
                         str(tmp_path / "cwrite"))
    rec = json.loads(capsys.readouterr().out)["mamba2p8b_layer"]
    assert rec["copy_fetch_factor"] == 2.0 and rec["copy_write_factor"] == 1.0
    assert rec["calls"] == 4 and rec["main_pass_launches"] == 4
    assert rec["main_pass_hbm_bytes_per_launch"] == (1000 * 2 + 500) * 1024
    assert rec["hbm_bytes_per_call"] == (1100 * 2 + 550) * 1024
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    import workloads as W
    assert rec["algorithmic_bytes"] == W.scan_bytes(W.spec("mamba2p8b_layer"))


def test_traffic_record_refuses_other_library_kernels(tmp_path):
    write_db(str(tmp_path / "cfetch"), "cfetch", [(COPY, [524288.0], 0, 1)], "FETCH_SIZE")
    write_db(str(tmp_path / "cwrite"), "cwrite", [(COPY, [1048576.0], 0, 1)], "WRITE_SIZE")
    rows = forward_run(2, 100.0, 1000.0)
    rows.append(("void mssm::state_update_kernel<16>(float*)", [5.0], 0, 1))
    write_db(str(tmp_path / "fetch"), "fetch", rows, "FETCH_SIZE")
    write_db(str(tmp_path / "write"), "write", forward_run(2, 50.0, 500.0), "WRITE_SIZE")
    with pytest.raises(RuntimeError, match="other kernels of the library"):
        bench.traffic_record("mamba2p8b_layer", 0, str(tmp_path / "fetch"),
                             str(tmp_path / "write"), str(tmp_path / "cfetch"),
                             str(tmp_path / "cwrite"))


def test_traffic_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    plan = {"segments": 4}
    assert bench.load_traffic("w", plan) is None  # no record
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "segments": 4,
           "main_pass_hbm_bytes_per_launch": 123, "hbm_bytes_per_call": 456}
    path.write_text(json.dumps({"w": rec}))
    assert bench.load_traffic("w", plan) == 123
    assert bench.load_traffic("w", plan, "hbm_bytes_per_call") == 456
    assert bench.load_traffic("other", plan) is None
    assert bench.load_traffic("w", {"segments": 2}) is None  # another plan
    path.write_text(json.dumps({"w": dict(rec, kernel_source_sha256_16="0" * 16)}))
    assert bench.load_traffic("w", plan) is None  # another kernel source


def test_hbm_and_alu_rooflines():
    r = bench.hbm_roofline(8e9, 1.0, "k", 1.0, traffic=9e9)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == 8000.0 and r["frac"] == 1.0 and r["traffic"] == 9e9
    r = bench.hbm_roofline(2e9, 1.0, "k", 1.0)
    assert r["frac"] == 0.25 and r["traffic"] is None
    # slots issued at the peak rate for 1 ms: fraction 1; bytes moved at 8 TB/s
    # in that time: the ALU ceiling is the HBM peak
    slots = bench.VALU_PEAK_TSLOTS * 1e12 * 1e-3
    a = bench.alu_figures(slots, 1.0, 8e9)
    assert a["frac"] == 1.0 and a["ceiling_frac_of_hbm_peak"] == 1.0
    a = bench.alu_figures(slots, 2.0, 4e9)
    assert a["frac"] == 0.5 and a["ceiling_frac_of_hbm_peak"] == 0.5


def test_call_breakdown_times_each_pack_and_scan(tmp_path, capsys):
    write_db(str(tmp_path / "kt"), "kt", forward_run(3, 1.0, 1.0), "FETCH_SIZE")
    bench.call_breakdown(str(tmp_path / "kt"))
    out = {l.split()[0]: float(l.split()[2]) for l in capsys.readouterr().out.splitlines()[1:]}
    assert out["pack_us"] == 3.0 and out["pack_to_scan_gap_us"] == 0.0
    assert out["scan_us"] == 197.0 and out["scan_to_next_pack_gap_us"] == 10.0


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stdout + p.stderr
