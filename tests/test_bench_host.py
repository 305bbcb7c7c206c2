"""Host-side logic of bench.py (no GPU): the one-GPU contract and the kernel
source hash that keys recorded counters."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // add one\n}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.source_hash()
    src.write_text("// a header comment\nint  f(int x) {\n\n  return x + 1;\n}\n")
    assert bench.source_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_hash() != h0


def test_traffic_record_requires_matching_source(tmp_path, monkeypatch):
    import json
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps({"w/default": {"source_sha": "nope", "bytes_per_launch": 1.0,
                                               "partition_avg_ns": 1000.0}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(table))
    assert bench.traffic_for("w", "default") == (None, None)
    table.write_text(json.dumps({"w/default": {"source_sha": bench.source_hash(),
                                               "bytes_per_launch": 5.0,
                                               "partition_avg_ns": 2500.0}}))
    assert bench.traffic_for("w", "default") == (5.0, 2.5)


def test_bench_workloads_build_names():
    assert "contig_b8" in bench.BENCH_WORKLOADS
    assert bench.bench_desc("paged_b64_xsplit").endswith("x-split pool layout")


def test_cpu_baseline_pool_reports_its_workers():
    import bench
    rec = bench.cpu_baseline("tiny_contig", budget_s=0.3)
    assert rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert 1 <= rec["cores"] <= bench.CPU_WORKERS_MAX
    assert rec["value"] > 0 and rec["seconds"] >= 0.3
    assert f"over {rec['cores']} worker processes" in rec["sample"]


def test_read_probe_library_validates_arguments():
    """The probe library loads and rejects bad arguments before any HIP call."""
    import ctypes
    import bench
    lib = ctypes.CDLL(bench.PROBE_LIB)
    f = lib.hbm_read_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    for mode in (0, 1, 2, 3):
        assert f(None, 1 << 20, 0, 0x10000, 64, mode, None) == 1      # no buffer
        assert f(0x10000, 1 << 20, 0, None, 64, mode, None) == 1      # no sink
        assert f(0x10000, 1 << 20, 0, 0x20000, 0, mode, None) == 1    # empty grid
        assert f(0x10000, 1000, 0, 0x20000, 64, mode, None) == 1      # not a multiple of 16
        assert f(0x10008, 1 << 20, 0, 0x20000, 64, mode, None) == 1   # misaligned
    assert f(0x10000, 1 << 20, 0, 0x20000, 64, 4, None) == 1          # unknown pattern
    assert f(0x10000, 1 << 20, 0, 0x20000, 64, -1, None) == 1         # unknown pattern


def test_cpu_baseline_leaves_no_child_process():
    import multiprocessing
    import psutil
    import bench
    before = {c.pid for c in psutil.Process().children(recursive=True)}
    rec = bench.cpu_baseline("tiny_contig", budget_s=0.2)
    assert rec["available_cores"] >= rec["cores"] >= 1
    assert rec["host_cores"] >= rec["available_cores"]
    assert not multiprocessing.active_children()
    after = {c.pid for c in psutil.Process().children(recursive=True)}
    assert after <= before, after - before
