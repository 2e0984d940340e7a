"""Host logic of bench.py, no GPU: the one-GPU refusal, which workloads a run
measures, the algorithmic byte count on hand-built cases, and the HBM traffic
bookkeeping from rocprofv3 counter files."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("workload,also,want", [
    (None, None, ("decode_down_gather", ["prefill_grouped_down", "gateup_gather",
                                          "router_gather", "mixed_grouped", "decode_layer",
                                          "decode_multi_gather"])),
    ("router_gather", None, ("router_gather", [])),
    ("prefill_grouped_down", None, ("prefill_grouped_down", [])),
    (None, "none", ("decode_down_gather", [])),
    (None, "prefill_grouped_down,decode_down_gather", ("decode_down_gather",
                                                       ["prefill_grouped_down"])),
    ("gateup_gather", "mixed_grouped", ("gateup_gather", ["mixed_grouped"])),
])
def test_resolve_workloads(workload, also, want):
    assert bench.resolve_workloads(workload, also) == want


def test_resolve_workloads_rejects_unknown():
    with pytest.raises(SystemExit):
        bench.resolve_workloads(None, "no_such_workload")


K, N, R = 16, 8, 4
PER_TOKEN = K * 2                  # one x row, bf16
PER_EXPERT = (R * K + N * R) * 2   # A_e and B_e, bf16
PER_ROW = N * 2 * 2                # base_out row read and written


def test_algorithmic_bytes_gather_hand_count():
    """3 tokens x top-2 = 6 rows; experts 0, 1 adapted, 2 packed with null
    cells (table length 3). Rows: (t0,e0) (t0,e1) (t1,e1) (t1,e5: past the
    table) (t2,e0) (t2,e2); token 2 is skipped by the map. Folded: rows 0-2,
    tokens {0, 1}, experts {0, 1}."""
    case = SimpleNamespace(path="gather", dtype="bf16", k_in=K, n_out=N, max_rank=R, top_k=2,
                           n_rows=6, n_tokens=3,
                           indices=np.array([0, 1, 1, 5, 0, 2], dtype=np.int32))
    tables = (np.array([16, 32, 0], np.uint64), np.array([16, 32, 0], np.uint64),
              np.ones(3, np.float32), 3)
    ra = np.array([1, 1, -1], dtype=np.int32)
    got = bench.algorithmic_traffic(case, tables, ra)
    want = 2 * PER_TOKEN + 2 * PER_EXPERT + 3 * PER_ROW + 4 * 6 + 4 * 3 + 20 * 3
    assert got == (want, 2 * 3 * R * (K + N), 6, 3, 1)
    # slot-major x: each of the 3 folded rows reads its own x row
    got = bench.algorithmic_traffic(case, tables, ra, x_by_row=True)
    assert got[0] == want + PER_TOKEN


def test_algorithmic_bytes_grouped_hand_count():
    """5 sorted rows, top-2 over 3 tokens; spans: expert 0 rows [0, 2), expert
    1 empty, expert 2 rows [2, 5); expert 1 has null cells; token 2 skipped.
    Windows of 3 rows: [0, 3) folds rows 0, 1 (e0, tokens 0, 1) and 2 (e2,
    token 0); [3, 5) folds row 3 (e2, token 1); row 4 (token 2) folds nothing."""
    import moe_expert_lora_amd as ml
    ml.load()
    case = SimpleNamespace(path="grouped", dtype="bf16", k_in=K, n_out=N, max_rank=R, top_k=2,
                           n_rows=5, n_tokens=3, n_route=3, cap=3,
                           expert_offsets=np.array([0, 2, 2, 5], dtype=np.int32),
                           sorted_ids=np.array([0, 3, 1, 2, 4], dtype=np.int32))
    tables = (np.array([16, 0, 48], np.uint64), np.array([16, 0, 48], np.uint64),
              np.ones(3, np.float32), 3)
    ra = np.array([1, 1, -1], dtype=np.int32)
    got = bench.algorithmic_traffic(case, tables, ra)
    meta = 4 * 3 + 4 * 4 + 20 * 3  # map, offsets, tables: per window
    w1 = 2 * PER_TOKEN + 2 * PER_EXPERT + 3 * PER_ROW + 4 * 3 + meta
    w2 = 1 * PER_TOKEN + 1 * PER_EXPERT + 1 * PER_ROW + 4 * 2 + meta
    assert got == (w1 + w2, 2 * 4 * R * (K + N), 5, 4, 2)


def test_algorithmic_bytes_grouped_by_launch_group():
    """The same 5 rows counted as one launch group [0, 5): tokens {0, 1} and
    experts {0, 2} are read once for the group."""
    case = SimpleNamespace(path="grouped", dtype="bf16", k_in=K, n_out=N, max_rank=R, top_k=2,
                           n_rows=5, n_tokens=3, n_route=3, cap=3,
                           expert_offsets=np.array([0, 2, 2, 5], dtype=np.int32),
                           sorted_ids=np.array([0, 3, 1, 2, 4], dtype=np.int32))
    tables = (np.array([16, 0, 48], np.uint64), np.array([16, 0, 48], np.uint64),
              np.ones(3, np.float32), 3)
    ra = np.array([1, 1, -1], dtype=np.int32)
    got = bench.algorithmic_traffic(case, tables, ra, groups=[(0, 5)])
    meta = 4 * 3 + 4 * 4 + 20 * 3
    want = 2 * PER_TOKEN + 2 * PER_EXPERT + 4 * PER_ROW + 4 * 5 + meta
    assert got == (want, 2 * 4 * R * (K + N), 5, 4, 1)


def test_algorithmic_bytes_grouped_unnamed_ids():
    """Sorted ids of -1 or past the last token fold nothing and read no x row."""
    case = SimpleNamespace(path="grouped", dtype="bf16", k_in=K, n_out=N, max_rank=R, top_k=2,
                           n_rows=4, n_tokens=2, n_route=2, cap=4,
                           expert_offsets=np.array([0, 2, 4], dtype=np.int32),
                           sorted_ids=np.array([0, -1, 4, 3], dtype=np.int32))
    tables = (np.array([16, 48], np.uint64), np.array([16, 48], np.uint64),
              np.ones(2, np.float32), 2)
    ra = np.array([1, 1], dtype=np.int32)
    got = bench.algorithmic_traffic(case, tables, ra, groups=[(0, 4)])
    want = 2 * PER_TOKEN + 2 * PER_EXPERT + 2 * PER_ROW + 4 * 4 + 4 * 2 + 4 * 3 + 20 * 2
    assert got == (want, 2 * 2 * R * (K + N), 4, 2, 1)


@pytest.mark.parametrize("n_rows,cap,want", [
    (32768, 8192, [(0, 16384), (16384, 32768)]),
    (16384, 8192, [(0, 16384)]),
    (12288, 8192, [(0, 12288)]),
    (50000, 20000, [(0, 20000), (20000, 40000), (40000, 50000)]),
    (100, 30, [(0, 100)]),
])
def test_all_windows_groups(n_rows, cap, want):
    assert bench.all_windows_groups(n_rows, cap) == want


def test_cpu_threads_respects_omp(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "3")
    assert bench.cpu_threads() == min(3, len(os.sched_getaffinity(0)))
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads() == len(os.sched_getaffinity(0))


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_from_scales_counters_by_the_copy(tmp_path, monkeypatch):
    """Two steps of a two-kernel fold: counters are summed over the fold's
    kernels, divided by the steps, and scaled by what the
    same counter reads for the plain copy of CALIB_BYTES (FETCH_SIZE reading
    half the copied bytes gives a factor 2)."""
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    k1, k2 = "mlora::shrink_kernel", "mlora::expand_kernel"
    _write_counters(tmp_path / "f", [(k1, "FETCH_SIZE", 100), (k2, "FETCH_SIZE", 300),
                                     (k1, "FETCH_SIZE", 100), (k2, "FETCH_SIZE", 300),
                                     ("other", "FETCH_SIZE", 9999)])
    _write_counters(tmp_path / "w", [(k1, "WRITE_SIZE", 10), (k2, "WRITE_SIZE", 50),
                                     (k1, "WRITE_SIZE", 10), (k2, "WRITE_SIZE", 50)])
    cal = bench.CALIB_BYTES / 1024.0
    _write_counters(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", cal / 2),
                                      ("fill", "FETCH_SIZE", 1)])
    _write_counters(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", cal)])
    bench.traffic_from("decode_down_gather", str(tmp_path / "f"), str(tmp_path / "w"),
                       str(tmp_path / "cf"), str(tmp_path / "cw"))
    rec = json.load(open(out))["decode_down_gather"]
    assert rec["fetch_kib_per_step"] == pytest.approx(400.0)
    assert rec["write_kib_per_step"] == pytest.approx(60.0)
    assert rec["copy_scale_fetch"] == pytest.approx(2.0)
    assert rec["copy_scale_write"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_step"] == pytest.approx((400.0 * 2 + 60.0) * 1024)
    assert rec["kernel_sha256_16"] == bench.kernel_hash()


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    inc = tmp_path / "k.inc"
    src.write_text("int a;  // one\n\n// two\nint b;\n")
    inc.write_text("int d;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src), str(inc)])
    h1 = bench.kernel_hash()
    src.write_text("int a;   // changed\n// more\n\nint b;\n")
    assert bench.kernel_hash() == h1
    src.write_text("int a;\nint c;\n")
    assert bench.kernel_hash() != h1
    # the included body counts too
    src.write_text("int a;  // one\n\n// two\nint b;\n")
    inc.write_text("int e;\n")
    assert bench.kernel_hash() != h1


def test_probe_library_exports_and_rejects_bad_arguments():
    """libmlora_probe.so (bench.py --probes) exports its four probes, and
    each rejects invalid arguments before any device call (so this runs on
    CPU)."""
    import ctypes
    lib = ctypes.CDLL(bench.PROBE_LIB)
    lib.mlora_probe_empty.restype = ctypes.c_int32
    lib.mlora_probe_empty.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.mlora_probe_read.restype = ctypes.c_int32
    lib.mlora_probe_read.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_void_p]
    us = ctypes.c_float()
    assert lib.mlora_probe_empty(0, ctypes.byref(us), ctypes.byref(us)) != 0
    assert lib.mlora_probe_empty(10, None, None) != 0
    for args in ((3, 4096, 12, 10), (-1, 4096, 12, 10), (0, 4095, 12, 10), (0, 8208, 12, 10), (0, 4100, 12, 10),
                 (1, 4096, 0, 10), (1, 4096, 33, 10), (1, 4096, 12, 0)):
        assert lib.mlora_probe_read(*args, ctypes.byref(us)) != 0, args
    assert lib.mlora_probe_read(0, 4096, 12, 10, None) != 0
    lib.mlora_probe_rmw.restype = ctypes.c_int32
    lib.mlora_probe_rmw.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p]
    for args in ((3, 0, 0, 10, 10), (-1, 0, 0, 10, 10), (0, 2, 0, 10, 10), (0, 0, 2, 10, 10),
                 (0, 0, 0, 0, 10), (0, 0, 0, 17, 10), (0, 0, 0, 10, 0)):
        assert lib.mlora_probe_rmw(*args, ctypes.byref(us)) != 0, args
    assert lib.mlora_probe_rmw(0, 0, 0, 10, 10, None) != 0
    lib.mlora_probe_stream.restype = ctypes.c_int32
    lib.mlora_probe_stream.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p]
    for args in ((0, 4, 4, 8, 8), (4097, 4, 4, 8, 8), (8, 2, 4, 8, 8), (8, 68, 4, 8, 8),
                 (8, 4, -4, 8, 8), (8, 4, 4, 0, 8), (8, 4, 4, 65, 8), (8, 4, 4, 8, 0),
                 (8, 4, 4, 8, 4097)):
        assert lib.mlora_probe_stream(*args, ctypes.byref(us)) != 0, args
    assert lib.mlora_probe_stream(8, 4, 4, 8, 8, None) != 0
