"""Host-side checks of bench.py: the byte and flop conventions behind its roofline
figures, the counter-summary arithmetic that turns rocprofv3 CSVs into the traffic
files under profiles/, the stale-counter guard, and the one-GPU contract."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_headline_bytes_and_flops():
    # B=8 H=16 L=4096 d=128 chunk 64: 1536 bytes per token-head plus a 64 KiB state per
    # head; per chunk C(C+1)(d_k+d_v) + 4 C d_k d_v flops over 64 chunks and 128 heads
    assert bench.prefill_bytes(8, 16, 4096, 128, 128) == 1536 * 8 * 16 * 4096 + 65536 * 128 == 813694976
    assert bench.prefill_flops(8, 16, 4096, 128, 128, 64) == 43083890688
    # a ragged tail chunk counts only its own rows
    full = bench.prefill_flops(1, 1, 128, 16, 16, 64)
    assert bench.prefill_flops(1, 1, 130, 16, 16, 64) == full + 2 * 3 * 32 + 4 * 2 * 16 * 16


def test_decode_step_bytes():
    # read and write the fp32 state, read q, k, v (bf16) and g (fp32), write o (bf16)
    assert bench.decode_step_bytes(256, 32, 128, 128) == 1086324736


def test_gate_modes_change_only_the_gate_bytes():
    kd = bench.prefill_bytes(1, 1, 10, 128, 128, gate="keydim")
    sc = bench.prefill_bytes(1, 1, 10, 128, 128, gate="scalar")
    no = bench.prefill_bytes(1, 1, 10, 128, 128, gate="none")
    assert kd - no == 10 * 128 * 4 and sc - no == 10 * 4


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name",
                               "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_calibration(tmp_path, monkeypatch):
    """The copy kernel moves 512 MiB each way; its counter readings fix bytes per
    counter unit, which then scale the kernel's readings (instances of one dispatch are
    summed, dispatches averaged)."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_ALL_FILE", str(tmp_path / "all.txt"))
    copy = "void at::native::elementwise_kernel<MulFunctor<float>>"
    dec = "_ZN3gla13decode_kernelIDF16bLi128ELi128ELb0EEEvNS_10DecodeArgsE"
    _write_counters(tmp_path / "cf", [dict(Dispatch_Id=1, Grid_Size=1, Kernel_Name=copy, Workgroup_Size=1,
                                           Counter_Name="FETCH_SIZE", Counter_Value=262144.0)])
    _write_counters(tmp_path / "cw", [dict(Dispatch_Id=1, Grid_Size=1, Kernel_Name=copy, Workgroup_Size=1,
                                           Counter_Name="WRITE_SIZE", Counter_Value=524288.0)])
    fetch = [dict(Dispatch_Id=d, Grid_Size=8192 * 256, Kernel_Name=dec, Workgroup_Size=256,
                  Counter_Name="FETCH_SIZE", Counter_Value=v) for d, v in ((1, 600.0), (1, 400.0), (2, 3000.0))]
    write = [dict(Dispatch_Id=1, Grid_Size=8192 * 256, Kernel_Name=dec, Workgroup_Size=256,
                  Counter_Name="WRITE_SIZE", Counter_Value=1000.0)]
    _write_counters(tmp_path / "f", fetch)
    _write_counters(tmp_path / "w", write)
    bench.summarize_traffic_all([str(tmp_path / x) for x in ("f", "w", "cf", "cw")], "cmd")
    line = [ln for ln in open(tmp_path / "all.txt") if ln.startswith("8192")][0].split()
    # fetch: (1000 + 3000) / 2 units x 2048 bytes; write: 1000 units x 1024 bytes
    assert line[1] == "2"
    assert float(line[2]) == pytest.approx(2000 * 2048 / 1e6, abs=0.05)
    assert float(line[3]) == pytest.approx(1000 * 1024 / 1e6, abs=0.05)


def test_stored_traffic_needs_the_current_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text("traffic_bytes_per_launch: 123\nkernel_source_sha256: %s\n" % bench.kernel_source_hash())
    assert bench.stored_traffic() == 123.0
    f.write_text("traffic_bytes_per_launch: 123\nkernel_source_sha256: %s\n" % ("0" * 64))
    assert bench.stored_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.stored_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
