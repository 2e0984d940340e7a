"""Benchmark of the MoE expert-LoRA fold on one MI355X.

One step = one pass of the fold over one synthetic batch: for the decode
workloads one mlora_gather_bgmv call, for the prefill workloads one
mlora_grouped_down_all call over every window of grouped_down_windows (with
--one-kernel: one mlora_grouped_down call per window). The host-side integer
work (tables, maps, windows) is done once before timing, as an engine does at
adapter install / batch setup; its cost is reported separately. Steps are
captured in HIP graphs and replayed (the fold reads its routing on the device
precisely so that it can be captured); eager launch cost is reported too.

Inputs are resident in HBM before timing starts. The steps cycle through
`copies` independent copies of x, A, B, base_out and the tables, so each step
reads data that no recent step touched (more bytes than L2 + MALL hold): the
figures are cold-cache HBM figures. Exactly --steps steps are timed.

Prints ONE JSON line (rank 0, N = 1) for the decode workload, with every other
full-size workload measured the same way under "also":
  value         rows covered per second (rows covered by the calls / wall time)
  roofline      algorithmic bytes per step / mean step time (HIP events on the
                replay stream) against the 8 TB/s HBM peak; a grouped step's
                bytes are counted per launch group of the all-windows call
                (also given per window); traffic = counter-measured HBM bytes
                per step from profiles/traffic.json when the kernel source
                still matches it, else null
  cpu_baseline  the fp64 CPU oracle timed on the host on a bounded sample,
                with the threads it used, the CPUs available and the model
  config        workload, rows, windows, kernel dispatches per step (counted
                in a captured step), copies
  copy_floor    torch's device copy moving the same bytes in one launch,
                replayed the same way: what one launch of that size streams
  warm_step_us  the same step replayed on one copy, inputs resident in L2 /
                MALL (context only: every other figure is cold HBM)
  hbm_copy_gbs  read + write GB/s of a plain 1 GiB device copy: a practical
                HBM figure for context (the roofline uses the nominal 8 TB/s)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA fold rows/s + achieved HBM GB/s (decode gather, prefill grouped)"
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "decode_down_gather"
# the workloads a default run measures: the decode line and, beside it, every
# other full-size workload (the tiny fp32 one is a parity case only)
MEASURED = ["decode_down_gather", "prefill_grouped_down", "gateup_gather", "router_gather",
            "mixed_grouped", "decode_layer", "decode_multi_gather"]
KERNEL_SOURCES = [os.path.join(ROOT, "moe_expert_lora_amd", "csrc", name)
                  for name in ("mlora_fold.hip", "mlora_resident_body.inc")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOAD_TEXT = {
    "tiny_gather_f32": "tiny gather fold f32: 4 tokens x top-2 of 4 experts, k_in 64, n_out 32, rank 8",
    "decode_down_gather": "Qwen3-MoE-like decode down-proj gather: 64 seqs x top-8 (640 rows padded), "
            "128 experts (96 adapted), k_in 768, n_out 2048, rank 16, bf16",
    "prefill_grouped_down": "prefill grouped down fold: 4096 tokens x top-8 (32768 sorted rows), Zipf(1.1) "
            "over 128 experts, k_in 768, n_out 2048, rank 32, bf16, windows of 8192",
    "gateup_gather": "gate/up gather: 256 seqs x top-8 (2048 rows), 128 experts, k_in 2048, "
            "n_out 768, rank 64, bf16",
    "router_gather": "router fold one-entry route: 8192 token rows, top_k 1, k_in 2048, n_out 128, "
             "rank 16, bf16",
    "mixed_grouped": "mixed prefill grouped fold: 16384 sorted rows, 256 experts (77 unadapted, "
             "duplicate ids), k_in 1536, n_out 4096, rank 16, bf16, windows of 8192",
    "decode_multi_gather": "decode down-proj gather (64 seqs x top-8, 640 rows, 128 experts, "
             "k_in 768, n_out 2048, rank 16) with 4 installed adapters, each adapting 96 "
             "experts; 6 Skip and 5 not-installed sequences; bf16",
    "decode_layer": "Qwen3-MoE-like decode layer, 64 seqs x top-8 (640 rows, 80 tokens), 128 "
             "experts (96 adapted): router one-entry route (k_in 2048, n_out 128), gate and up "
             "(k_in 2048, n_out 768, fused output) in one set, down on slot-major x (k_in 768, "
             "n_out 2048); rank 16, bf16",
}


def kernel_hash() -> str:
    """Hash of the kernel sources' code (mlora_fold.hip, then the decode
    kernel's body that it includes): line comments and blank lines are dropped
    first, so an edit of the comments keeps recorded counters valid."""
    code = []
    for path in KERNEL_SOURCES:
        with open(path) as f:
            for line in f:
                line = line.split("//", 1)[0].rstrip()
                if line:
                    code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes: what the fold must move, counted from the inputs
# ---------------------------------------------------------------------------

def all_windows_groups(n_rows, cap, min_rows=16384):
    """Row ranges of the launches of mlora_grouped_down_all (its header): whole
    windows of `cap` rows, at least `min_rows` rows per launch."""
    m = 1 if cap >= min_rows else -(-min_rows // cap)
    chunk = cap * m
    return [(s, min(s + chunk, n_rows)) for s in range(0, n_rows, chunk)]


def algorithmic_traffic(case, tables, row_adapter, groups=None, x_by_row=False):
    """(bytes, flops, rows, folded_rows, units) per step, summed over units.

    A unit is one call's worth of rows that reads its own operands: the whole
    call for a gather (x_by_row: each row reads its own x row, so x counts per
    folded row), and for a grouped step each row range of `groups`
    (default: the windows of grouped_down_windows). Per unit:
    bytes = unique tokens * k_in * 2 + unique experts * (r*k_in + n_out*r) * 2
          + folded rows * n_out * 2 * 2 (base_out read + write)
          + 4 * rows (indices / sorted_ids) + 4 * tokens (map)
          + 4 * (n_route + 1) (offsets, grouped) + 20 * n_experts (tables)
    A grouped row folds when it lies in an adapted expert's span and its
    sorted id names a token whose map entry is >= 0.
    """
    at, bt, _, n_exp = tables
    elt = 2 if case.dtype == "bf16" else 4
    K, N, R = case.k_in, case.n_out, case.max_rank
    live_cell = np.zeros(max(n_exp, 1), dtype=bool)
    if n_exp:
        live_cell[:n_exp] = (at != 0) & (bt != 0)
    ra = np.asarray(row_adapter)

    def cell_ok(e):
        return (e >= 0) & (e < n_exp) & live_cell[np.clip(e, 0, max(n_exp - 1, 0))]

    units = []
    if case.path == "gather":
        rows = np.arange(case.n_rows)
        tok = rows // case.top_k
        e = case.indices.astype(np.int64)
        live = (ra[tok] >= 0) & cell_ok(e)
        # x rows read: the tokens', or (slot-major x) the rows' own
        xrow = rows if x_by_row else tok
        units.append((case.n_rows, xrow[live], e[live], 0))
    else:
        off = case.expert_offsets.astype(np.int64)
        owner = np.searchsorted(off, np.arange(case.n_rows), side="right") - 1
        ids = case.sorted_ids.astype(np.int64)
        named = (ids >= 0) & (ids // case.top_k < case.n_tokens)
        tok_all = np.where(named, ids // case.top_k, 0)
        inside = (owner >= 0) & (owner < len(off) - 1)
        if groups is None:
            import moe_expert_lora_amd as ml
            groups = ml.mlora_grouped_down_windows(case.n_rows, case.cap)
        for (s, t) in groups:
            o = owner[s:t]
            tk = tok_all[s:t]
            live = inside[s:t] & named[s:t] & cell_ok(o) & (ra[np.clip(tk, 0, len(ra) - 1)] >= 0)
            units.append((t - s, tk[live], o[live], case.n_route + 1))
    total_b = 0
    flops = 0
    folded = 0
    rows_total = 0
    for (rows, toks, exps, n_off) in units:
        f = toks.shape[0]
        b = (np.unique(toks).size * K * elt + np.unique(exps).size * (R * K + N * R) * elt
             + f * N * elt * 2 + 4 * rows + 4 * len(ra) + 4 * n_off + 20 * n_exp)
        total_b += int(b)
        flops += 2 * f * R * (K + N)
        folded += f
        rows_total += rows
    return total_b, flops, rows_total, folded, len(units)


# ---------------------------------------------------------------------------
# device staging with rotating copies
# ---------------------------------------------------------------------------

class Staged:
    def __init__(self, case, copies, device="cuda", two_kernel=True):
        import torch
        from staging import DeviceCase
        self.case = case
        self.primary = DeviceCase(case, device, two_kernel=two_kernel)
        if two_kernel:
            # one workspace, allocated before any capture, shared by every copy
            self.primary.workspace_for(getattr(self.primary, "windows", None))
        self.copies = [self.primary]
        for _ in range(copies - 1):
            self.copies.append(self.primary_clone(device))
        self.bases = [c.base0.clone() for c in self.copies]
        torch.cuda.synchronize()

    def primary_clone(self, device):
        """Same data at new addresses (weights, x, base_out and the tables)."""
        import copy
        import moe_expert_lora_amd as ml
        from staging import u64_to_device
        p = self.primary
        c = copy.copy(p)
        c.x = p.x.clone()
        c.a_pool = p.a_pool.clone()
        c.b_pool = p.b_pool.clone()
        c.base0 = p.base0.clone()
        at, bt, st, n = p.tables_host
        da = c.a_pool.data_ptr() - p.a_pool.data_ptr()
        db = c.b_pool.data_ptr() - p.b_pool.data_ptr()
        at2 = np.where(at != 0, at + np.uint64(da % (1 << 64)), 0).astype(np.uint64)
        bt2 = np.where(bt != 0, bt + np.uint64(db % (1 << 64)), 0).astype(np.uint64)
        c.a_table = u64_to_device(np.concatenate([at2, [0]]), device)
        c.b_table = u64_to_device(np.concatenate([bt2, [0]]), device)
        c.scale_table = p.scale_table.clone()
        c.route = ml.make_route(c.a_table, c.b_table, c.scale_table, n, self.case.k_in,
                                self.case.n_out, self.case.max_rank, p.tdtype)
        c.tables_host = (at2, bt2, st, n)
        return c

    def step(self, i):
        k = i % len(self.copies)
        self.copies[k].fold(self.bases[k])


def copy_bytes(case):
    elt = 2 if case.dtype == "bf16" else 4
    return (case.x.size + case.a_pool.size + case.b_pool.size + case.base.size) * elt


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    """Host threads the CPU leg uses: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when that is set (the host's share of cores)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def cpu_baseline(case, budget_s=10.0):
    """The fp64 oracle (per-expert NumPy matmuls) timed on the host: rows
    covered per second and the algorithmic bytes of the sample per second."""
    import oracle
    from oracle.case import OracleView, to_f64
    from threadpoolctl import threadpool_limits

    threads = cpu_threads()
    view = OracleView(case)
    base64 = to_f64(case.base, case.dtype)
    tables = (np.asarray(view.a_table, np.uint64), np.asarray(view.b_table, np.uint64),
              None, view.n_experts)
    if case.path == "gather":
        def run():
            return oracle.fold_gather(view.x, view.a_table, view.b_table, view.scale_table,
                                      view.mats, base64, case.indices, view.row_adapter,
                                      case.top_k)
        rows_per = case.n_rows
        groups = None
        sample = f"the full {case.name} call ({rows_per} rows)"
    else:
        # bounded sample: the first window
        s, e = oracle.grouped_down_windows(case.n_rows, case.cap)[0]

        def run():
            return oracle.fold_grouped(view.x, view.a_table, view.b_table, view.scale_table,
                                       view.mats, base64, case.expert_offsets, case.sorted_ids,
                                       view.row_adapter, case.top_k, s, e)
        rows_per = e - s
        groups = [(s, e)]
        sample = f"the first window [{s}, {e}) of {case.name}"
    sample_bytes = algorithmic_traffic(case, tables, view.row_adapter, groups)[0]
    with threadpool_limits(limits=threads):
        run()  # warm-up
        t0 = time.perf_counter()
        iters = 0
        while True:
            run()
            iters += 1
            el = time.perf_counter() - t0
            if (el >= budget_s and iters >= 3) or el >= 3 * budget_s:
                break
    return {"value": rows_per * iters / el, "unit": "rows/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{sample}, {iters}x in {el:.1f} s (fp64 NumPy, per-expert matmuls, "
                      f"BLAS limited to {threads} threads)",
            "gbs": sample_bytes * iters / el / 1e9,
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counter runs
# ---------------------------------------------------------------------------

CALIB_BYTES = 1 << 29  # 512 MiB copied by --calibrate-copy


def calibrate_copy():
    """A plain device copy of CALIB_BYTES (read CALIB_BYTES, write CALIB_BYTES);
    run under `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` to scale the
    counters of the fold runs."""
    import torch
    src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": CALIB_BYTES}), flush=True)


PROBE_LIB = os.path.join(ROOT, "moe_expert_lora_amd", "libmlora_probe.so")


def probes():
    """The floors that bound one launch of the fold (libmlora_probe.so, built
    with the fold library): an empty launch, eager and in a HIP graph; the
    read rate of 8192 rows of 4096 bytes (a k_in = 2048 bf16 operand) in
    the folds' MFMA-operand pattern (16 rows x 64 bytes per wave
    instruction), row-contiguously (1 KB of one row per instruction) and
    row-contiguously straight into LDS, read back there in the operand
    pattern, at row strides of 4096 bytes (dense rows), 4160 and 8192; and the
    read-modify-write rate of a 64 MiB bf16 buffer in the grouped expand's
    wave tile, by rows and by contiguous workgroup blocks, with the units in
    block order or each XCD on a contiguous eighth, plain or non-temporal;
    and launches shaped like the decode fold (192 or 256 workgroups, each
    streaming its own weights and read-modify-writing its own rows, no
    dependent load), replayed in a HIP graph: the floor of one such launch."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"bench.py: {PROBE_LIB} is missing; build with "
                         "python -m moe_expert_lora_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.mlora_probe_empty.restype = ctypes.c_int32
    lib.mlora_probe_empty.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                                      ctypes.POINTER(ctypes.c_float)]
    lib.mlora_probe_read.restype = ctypes.c_int32
    lib.mlora_probe_read.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.POINTER(ctypes.c_float)]
    eager, graph = ctypes.c_float(), ctypes.c_float()
    rc = lib.mlora_probe_empty(1000, ctypes.byref(eager), ctypes.byref(graph))
    if rc:
        raise SystemExit(f"bench.py: mlora_probe_empty failed (HIP error {rc})")
    out = {"empty_launch_us": {"eager": eager.value, "graph": graph.value}, "read": []}
    useful = 8192 * 4096
    for name, pattern in (("operand", 0), ("rows", 1), ("rows_via_lds", 2)):
        for stride in (4096, 4160, 8192):
            us = ctypes.c_float()
            rc = lib.mlora_probe_read(pattern, stride, 12, 240, ctypes.byref(us))
            if rc:
                raise SystemExit(f"bench.py: mlora_probe_read failed (HIP error {rc})")
            out["read"].append({"pattern": name, "row_stride": stride, "us": us.value,
                                "gbs": useful / (us.value * 1e-6) / 1e9})
            print(json.dumps(out["read"][-1]), file=sys.stderr, flush=True)
    out["read_bytes"] = useful
    # read-modify-write of a 64 MiB bf16 buffer (one prefill launch group's
    # base_out), 10 buffers rotated past MALL
    lib.mlora_probe_rmw.restype = ctypes.c_int32
    lib.mlora_probe_rmw.argtypes = [ctypes.c_int32] * 5 + [ctypes.POINTER(ctypes.c_float)]
    rmw_bytes = 2 * 16384 * 4096
    out["rmw"] = []
    for name, pattern in (("tile", 0), ("row", 1), ("flat", 2)):
        for xcdc in (0, 1):
            for nt in (1, 0):
                us = ctypes.c_float()
                rc = lib.mlora_probe_rmw(pattern, xcdc, nt, 10, 40, ctypes.byref(us))
                if rc:
                    raise SystemExit(f"bench.py: mlora_probe_rmw failed (HIP error {rc})")
                out["rmw"].append({"pattern": name, "xcd_contiguous": bool(xcdc),
                                   "non_temporal": bool(nt), "us": us.value,
                                   "gbs": rmw_bytes / (us.value * 1e-6) / 1e9})
                print(json.dumps(out["rmw"][-1]), file=sys.stderr, flush=True)
    out["rmw_bytes"] = rmw_bytes
    # launches shaped like the decode fold with no dependent load: each
    # workgroup reads its own weight bytes and reads-modifies-writes its own
    # rows; 64 buffer sets rotated (>= 640 MB), replayed in a HIP graph
    lib.mlora_probe_stream.restype = ctypes.c_int32
    lib.mlora_probe_stream.argtypes = [ctypes.c_int32] * 5 + [ctypes.POINTER(ctypes.c_float)]
    out["stream"] = []
    for units, w_kb, r_kb in ((192, 44, 8), (256, 32, 8), (192, 0, 0)):
        us = ctypes.c_float()
        rc = lib.mlora_probe_stream(units, w_kb, r_kb, 64, 256, ctypes.byref(us))
        if rc:
            raise SystemExit(f"bench.py: mlora_probe_stream failed (HIP error {rc})")
        moved = units * (w_kb + 2 * r_kb) * 1024
        out["stream"].append({"workgroups": units, "weight_kb": w_kb, "row_kb_rmw": r_kb,
                              "bytes": moved, "us": us.value,
                              "gbs": moved / (us.value * 1e-6) / 1e9})
        print(json.dumps(out["stream"][-1]), file=sys.stderr, flush=True)
    return out


def copy_bandwidth(n_bytes=1 << 30, reps=10):
    """Read + write GB/s of a plain device copy of n_bytes (torch's copy kernel),
    timed with HIP events on the current stream: a practical HBM figure beside
    the nominal peak, reported for context and never used as the roofline."""
    import torch
    src = torch.empty(n_bytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n_bytes / sec / 1e9


def _pmc_rows(path):
    import csv
    rows = []
    for root, _, files in os.walk(path):
        for f in files:
            if f.endswith("counter_collection.csv"):
                rows.extend(csv.DictReader(open(os.path.join(root, f))))
    return rows


def _mean_counter(rows, counter, match):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def _tables_and_map(case):
    """Host tables (fake nonzero addresses stand in for the device weights; only
    which cells are null matters here) and the row map of a workload, from the
    library's host functions."""
    import moe_expert_lora_amd as ml
    import workloads
    ids = np.array([e for (e, _, _, _) in case.entries], dtype=np.int32)
    a = np.array([0 if h == workloads.NULL_HANDLE else 16 * (h + 1)
                  for (_, h, _, _) in case.entries], dtype=np.uint64)
    b = np.array([0 if h == workloads.NULL_HANDLE else 16 * (h + 1)
                  for (_, _, h, _) in case.entries], dtype=np.uint64)
    sc = np.array([s for (_, _, _, s) in case.entries], dtype=np.float32)
    packed = ml.mlora_pack_expert_tables(ids, a, b, sc)
    tables = packed if packed is not None else (np.zeros(0, np.uint64), np.zeros(0, np.uint64),
                                                 np.zeros(0, np.float32), 0)
    if case.map_kind == "decode":
        ra = ml.mlora_build_moe_row_adapter_decode(case.adapter_slots, case.padded_n,
                                                   case.active, case.has_moe_lora)
    else:
        ra = ml.mlora_build_moe_row_adapter_host(case.cu_seqlens, case.stream_slots)
    full = np.full(max(case.n_tokens, ra.shape[0]), -1, dtype=np.int32)
    full[: ra.shape[0]] = ra
    return tables, full


def recorded_traffic(workload):
    """Counter-measured HBM bytes per step of `workload` from profiles/
    traffic.json, or None when there is no record or the kernel source has
    changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(workload)
    except (OSError, ValueError):
        return None
    if rec and rec.get("kernel_sha256_16") == kernel_hash():
        return rec.get("hbm_bytes_per_step")
    return None


def traffic_from(workload, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """Per-step HBM bytes of the fold from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch) of `bench.py --counters`, each scaled by what the counter reads
    for the plain copy of CALIB_BYTES; recorded in profiles/traffic.json with
    the kernel hash.

    A step runs one or more fold kernels (a shrink and an expand; the
    pipelined grouped call adds one launch per later group of windows).
    Every kernel runs at least once per step, so the least frequent one
    counts the steps, and the per-step figure is the counters summed over all
    fold dispatches divided by that count."""
    is_copy = lambda n: "mlora" not in n  # noqa: E731
    rows_f, rows_w = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    names = sorted({r["Kernel_Name"] for r in rows_f + rows_w if "mlora" in r["Kernel_Name"]})

    def per_step(rows, counter):
        vals = {n: [float(r["Counter_Value"]) for r in rows
                    if r["Counter_Name"] == counter and r["Kernel_Name"] == n] for n in names}
        vals = {n: v for n, v in vals.items() if v}
        steps = min(len(v) for v in vals.values())
        total = sum(sum(v) for v in vals.values())
        return total / steps, [len(v) for v in vals.values()]

    f_kib, nf = per_step(rows_f, "FETCH_SIZE")
    w_kib, nw = per_step(rows_w, "WRITE_SIZE")
    cal_rows_f = _pmc_rows(cal_fetch_dir)
    cal_rows_w = _pmc_rows(cal_write_dir)
    # the copy dispatch is the largest FETCH_SIZE / WRITE_SIZE in the calibration runs
    cf = max(float(r["Counter_Value"]) for r in cal_rows_f
             if r["Counter_Name"] == "FETCH_SIZE" and is_copy(r["Kernel_Name"]))
    cw = max(float(r["Counter_Value"]) for r in cal_rows_w
             if r["Counter_Name"] == "WRITE_SIZE" and is_copy(r["Kernel_Name"]))
    kf = CALIB_BYTES / (cf * 1024.0)
    kw = CALIB_BYTES / (cw * 1024.0)
    rec = {
        "kernel_sha256_16": kernel_hash(),
        "fetch_kib_per_step": f_kib, "write_kib_per_step": w_kib,
        "kernels": [re.sub(r"(?<=>)\(.*$", "", n.replace("void mlora::(anonymous namespace)::", ""))
                    for n in names],
        "dispatches": [nf, nw],
        "copy_scale_fetch": kf, "copy_scale_write": kw,
        "hbm_bytes_per_step": f_kib * 1024.0 * kf + w_kib * 1024.0 * kw,
    }
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: rec}))


# ---------------------------------------------------------------------------
# HIP graphs: capture, and the kernel dispatches one captured step holds
# ---------------------------------------------------------------------------

def _hip_runtime():
    """The HIP runtime library this process already loaded (PyTorch's)."""
    import ctypes
    with open("/proc/self/maps") as f:
        paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    if not paths:
        return None
    lib = ctypes.CDLL(sorted(paths)[0])
    lib.hipGraphGetNodes.restype = ctypes.c_int
    lib.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.hipGraphNodeGetType.restype = ctypes.c_int
    lib.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    return lib


def _new_graph(keep=False):
    import torch
    if keep:
        try:
            return torch.cuda.CUDAGraph(keep_graph=True)
        except TypeError:
            return None
    return torch.cuda.CUDAGraph()


def capture(fn, keep=False):
    """A HIP graph of whatever `fn` enqueues on the current stream (captured
    on a side stream, as torch requires)."""
    import torch
    g = _new_graph(keep)
    if g is None:
        return None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def kernel_nodes(g):
    """Kernel nodes of a captured graph (hipGraphNodeTypeKernel == 0), or None
    when the runtime or torch does not expose the graph."""
    import ctypes
    try:
        lib = _hip_runtime()
        raw = g.raw_cuda_graph()
        n = ctypes.c_size_t(0)
        if lib is None or lib.hipGraphGetNodes(ctypes.c_void_p(raw), None, ctypes.byref(n)):
            return None
        nodes = (ctypes.c_void_p * n.value)()
        if lib.hipGraphGetNodes(ctypes.c_void_p(raw), nodes, ctypes.byref(n)):
            return None
        kinds = ctypes.c_int(-1)
        count = 0
        for i in range(n.value):
            if lib.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(kinds)) == 0 \
                    and kinds.value == 0:
                count += 1
        return count
    except Exception:  # pragma: no cover - depends on the runtime
        return None


class Rotation:
    """`steps` steps of a rotation over `copies` copies as HIP graphs: one
    graph of a whole rotation, replayed, and one of the remaining steps (the
    first `steps % copies` copies), so exactly `steps` steps run."""

    def __init__(self, step, copies, steps, eager=False):
        self.full = steps // copies
        self.rem = steps % copies
        self.eager = eager
        self.step, self.copies = step, copies
        if not eager:
            self.g_full = capture(lambda: [step(i) for i in range(copies)]) if self.full else None
            self.g_rem = capture(lambda: [step(i) for i in range(self.rem)]) if self.rem else None

    def run(self):
        if self.eager:
            for _ in range(self.full):
                for i in range(self.copies):
                    self.step(i)
            for i in range(self.rem):
                self.step(i)
            return
        for _ in range(self.full):
            self.g_full.replay()
        if self.g_rem is not None:
            self.g_rem.replay()


def copy_floor(n_bytes, steps, device="cuda"):
    """A plain device copy that moves `n_bytes` (half read, half written) in
    one launch: torch's copy kernel, graph-replayed over enough rotating
    buffer pairs that every copy reads cold HBM. Returns (us per copy, GB/s)."""
    import torch
    half = max(256, (int(n_bytes) // 2 + 255) // 256 * 256)
    pairs = max(2, min(256, math.ceil(640e6 / (2 * half))))
    src = [torch.ones(half // 2, dtype=torch.bfloat16, device=device) for _ in range(pairs)]
    dst = [torch.empty_like(t) for t in src]
    torch.cuda.synchronize()
    rot = Rotation(lambda i: dst[i].copy_(src[i]), pairs, steps)
    rot.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    rot.run()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del src, dst, rot
    torch.cuda.empty_cache()
    return us, 2 * half / (us * 1e-6) / 1e9


def host_loop(st, steps):
    """The host-loop baseline on a staged grouped workload: each step copies
    expert_offsets to the host (a synchronisation) and makes one grouped
    launch per adapted expert's span (mlora_apply_expert_lora_sorted), cycling
    through the same rotating copies. Eager by nature; wall clock per step."""
    import torch
    import moe_expert_lora_amd as ml
    case = st.case
    off0 = st.primary.offsets.cpu().numpy().astype(np.int64)
    ws = None
    if st.primary.two_kernel and case.dtype == "bf16":
        need = ml.mlora_grouped_down_workspace_bytes(0, int(np.diff(off0).max()), case.max_rank)
        ws = torch.empty(max(256, need), dtype=torch.uint8, device="cuda")
    at0, bt0, _, n = st.primary.tables_host
    launched = sum(1 for e in range(min(len(off0) - 1, n))
                   if off0[e + 1] > off0[e] and at0[e] != 0 and bt0[e] != 0)

    def step(i):
        c = st.copies[i % len(st.copies)]
        off_h = c.offsets.cpu().numpy()  # the device-to-host copy: waits for the stream
        at, bt, _, _ = c.tables_host
        ml.mlora_apply_expert_lora_sorted(c.route, c.x, st.bases[i % len(st.copies)], c.offsets,
                                          off_h, at, bt, c.sorted_ids, c.row_adapter,
                                          case.top_k, workspace=ws)

    for i in range(min(3, steps)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    return {"us_per_step": us, "rows_per_s": case.n_rows / (us * 1e-6),
            "kernel_launches_per_step": launched * (2 if ws is not None else 1),
            "what": "mlora_apply_expert_lora_sorted: offsets copied to the host each step, "
                    "then one grouped launch per adapted expert's span (eager, wall clock); "
                    "a baseline for what device-side routing buys, not a target"}


def measure(workload, args, cpu_seconds):
    """One workload: stage it, time exactly `args.steps` graph-replayed steps,
    and return the result record (the JSON line's fields)."""
    import torch
    import moe_expert_lora_amd as ml
    import workloads

    case = workloads.WORKLOADS[workload]()
    cb = copy_bytes(case)
    copies = args.copies or max(2, min(64, math.ceil(640e6 / cb)))
    st = Staged(case, copies, two_kernel=not args.one_kernel)
    tables = st.primary.tables_host
    ra = st.primary.row_adapter_host
    windows = 1
    groups = None
    if case.path == "grouped":
        windows = len(ml.mlora_grouped_down_windows(case.n_rows, case.cap))
        if not args.one_kernel and case.dtype == "bf16":
            groups = all_windows_groups(case.n_rows, case.cap)
    alg_bytes, flops, rows, folded, units = algorithmic_traffic(case, tables, ra, groups)
    win_bytes = algorithmic_traffic(case, tables, ra)[0]

    # host-side integer work of one batch, timed for the record
    t0 = time.perf_counter()
    for _ in range(50):
        if case.map_kind == "decode":
            ml.mlora_build_moe_row_adapter_decode(case.adapter_slots, case.padded_n, case.active,
                                                  case.has_moe_lora)
        else:
            ml.mlora_build_moe_row_adapter_host(case.cu_seqlens, case.stream_slots)
        if case.path == "grouped":
            ml.mlora_grouped_down_windows(case.n_rows, case.cap)
    host_us = (time.perf_counter() - t0) / 50 * 1e6

    for i in range(args.warmup):
        st.step(i)
    torch.cuda.synchronize()
    dispatches = None
    if not args.eager:
        one = capture(lambda: st.step(0), keep=True)
        dispatches = kernel_nodes(one) if one is not None else None
        del one
    # The fold reads its routing on the device, so a step is captured in a
    # HIP graph and replayed, as a decode loop runs it; the steps cycle
    # through the copies so that each one reads cold HBM.
    steps = args.steps
    rot = Rotation(st.step, copies, steps, eager=args.eager)
    rot.run()  # one untimed pass of the graphs themselves
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, wall clock and HIP events on the
    # stream the graphs replay on
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    rot.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = e0.elapsed_time(e1) * 1e3 / steps

    out_extra = {}
    if not args.counters:
        # spread: per-rotation duration over a second pass of whole rotations
        if not args.eager and rot.full:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(max(3, rot.full))]
            for a, b in ev:
                a.record(stream)
                rot.g_full.replay()
                b.record(stream)
            torch.cuda.synchronize()
            dur = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3 / copies
            out_extra["step_us_p10_p50_p90"] = [float(np.percentile(dur, q)) for q in (10, 50, 90)]
        # eager launches (host launch path included), for the record
        t1 = time.perf_counter()
        for i in range(copies):
            st.step(i)
        torch.cuda.synchronize()
        out_extra["eager_step_us"] = (time.perf_counter() - t1) / copies * 1e6
        # warm figure, for context: one copy's step, captured as many times
        # as a rotation holds steps and replayed, inputs resident in L2 / MALL
        if not args.eager:
            wg = capture(lambda: [st.step(0) for _ in range(copies)])
            wg.replay()
            torch.cuda.synchronize()
            w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = max(1, math.ceil(steps / copies))
            w0.record(stream)
            for _ in range(reps):
                wg.replay()
            w1.record(stream)
            torch.cuda.synchronize()
            out_extra["warm_step_us"] = w0.elapsed_time(w1) * 1e3 / (reps * copies)
            del wg
        if case.path == "grouped" and not args.eager:
            out_extra["host_loop_baseline"] = host_loop(st, min(steps, 50))
        fl_us, fl_gbs = copy_floor(alg_bytes, steps)
        out_extra["copy_floor"] = {
            "us": fl_us, "gbs": fl_gbs,
            "what": "torch's device copy moving the step's algorithmic bytes (half read, "
                    "half written) in one launch, graph-replayed over rotating buffers"}
    del rot, st
    torch.cuda.empty_cache()

    achieved = alg_bytes / (step_us * 1e-6) / 1e9
    traffic = recorded_traffic(workload)

    cpu = cpu_baseline(case, cpu_seconds) if cpu_seconds > 0 else None
    unit = ("one mlora_gather_bgmv call" if case.path == "gather" else
            f"one mlora_grouped_down_all call over {windows} windows"
            if groups is not None else f"{windows} mlora_grouped_down calls (one per window)")
    out = {
        "metric": METRIC,
        "value": rows * steps / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": wall / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if case.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generators; random-init adapter weights)",
        "config": {
            "workload": f"{workload}: {WORKLOAD_TEXT[workload]}",
            "path": case.path,
            "rows_per_step": rows,
            "folded_rows_per_step": folded,
            "windows_per_step": windows,
            "kernel_dispatches_per_step": dispatches,
            "workspace": not args.one_kernel,
            "rotating_copies": copies,
            "timing": ("eager launches" if args.eager else
                       "HIP graphs of whole rotations over the copies plus the remainder, "
                       "replayed; HIP events on the replay stream"),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "unit_of_work": unit,
            "algorithmic_bytes": alg_bytes,
            "bytes_counted_by": ("the call" if case.path == "gather" else
                                 f"{units} launch groups" if groups is not None else
                                 f"{units} windows"),
            "algorithmic_bytes_by_window": win_bytes,
            "flops": flops,
            "step_us_mean": step_us,
        },
        "cpu_baseline": cpu,
        "host_setup_us": host_us,
        "notes": "the pages quote no performance numbers; vs_baseline is null",
    }
    out["roofline"].update({k: v for k, v in out_extra.items() if k == "step_us_p10_p50_p90"})
    out.update({k: v for k, v in out_extra.items() if k != "step_us_p10_p50_p90"})
    return out


def measure_layer(args, cpu_seconds):
    """A decode layer's LoRA folds at the decode batch (workloads.
    decode_layer_cases): the router's one-entry route, gate and up into the
    two halves of one fused output, and down on slot-major x. The layer step
    is three launches, as an engine orders them (router fold before the
    top-k; gate and up in one projection set after their base product; down
    after the activation); the same folds as four separate calls are timed
    beside it, and each fold alone."""
    import torch
    import moe_expert_lora_amd as ml
    import workloads

    cases = workloads.decode_layer_cases()
    router, gate, up, down = cases
    tot = sum(copy_bytes(c) for c in cases)
    copies = args.copies or max(2, min(64, math.ceil(640e6 / tot)))
    st = {c.name: Staged(c, copies, two_kernel=False) for c in cases}
    inter = gate.n_out
    fused = [torch.cat([st["gate"].bases[k], st["up"].bases[k]], dim=1).contiguous()
             for k in range(copies)]

    def proj(name, k, out, x_by_row=False):
        c = st[name].copies[k]
        return ml.make_projection(c.route, c.x, out, c.indices, c.row_adapter,
                                  st[name].case.top_k, x_by_row=x_by_row)

    P = {"router": [proj("router", k, st["router"].bases[k]) for k in range(copies)],
         "gate": [proj("gate", k, fused[k][:, :inter]) for k in range(copies)],
         "up": [proj("up", k, fused[k][:, inter:]) for k in range(copies)],
         "down": [proj("down", k, st["down"].bases[k], True) for k in range(copies)]}
    torch.cuda.synchronize()
    steps = args.steps
    stream = torch.cuda.current_stream()

    def timed(step):
        rot = Rotation(step, copies, steps)
        rot.run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        rot.run()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        del rot
        return e0.elapsed_time(e1) * 1e3 / steps, wall / steps * 1e3

    def layer_step(k):
        ml.mlora_gather_bgmv_set([P["router"][k]])
        ml.mlora_gather_bgmv_set([P["gate"][k], P["up"][k]])
        ml.mlora_gather_bgmv_set([P["down"][k]])

    def calls_step(k):
        for n in ("router", "gate", "up", "down"):
            ml.mlora_gather_bgmv_set([P[n][k]])

    layer_us, layer_ms = timed(layer_step)
    if args.counters:
        calls_us, alone = None, {}
    else:
        calls_us, _ = timed(calls_step)
        alone = {n: timed(lambda k, n=n: ml.mlora_gather_bgmv_set([P[n][k]]))[0]
                 for n in ("router", "gate", "up", "down")}
    nbytes = {}
    rows = 0
    for c in cases:
        tables, ra = _tables_and_map(c)
        b, _, r, _, _ = algorithmic_traffic(c, tables, ra, x_by_row=c.notes.get("x_rows") == "row")
        nbytes[c.name] = b
        rows += r
    total = sum(nbytes.values())
    del st, fused, P
    torch.cuda.empty_cache()

    cpu = None
    if cpu_seconds > 0:
        import oracle
        from oracle.case import OracleView, to_f64
        from threadpoolctl import threadpool_limits
        views = [(OracleView(c), to_f64(c.base, c.dtype), c) for c in cases]
        threads = cpu_threads()

        def run():
            for v, b, c in views:
                oracle.fold_gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, b,
                                   c.indices, v.row_adapter, c.top_k,
                                   x_rows=c.notes.get("x_rows", "token"))
        with threadpool_limits(limits=threads):
            run()
            t0 = time.perf_counter()
            it = 0
            while True:
                run()
                it += 1
                el = time.perf_counter() - t0
                if (el >= cpu_seconds and it >= 3) or el >= 3 * cpu_seconds:
                    break
        cpu = {"value": rows * it / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
               "sample": f"the four folds of one decode layer, {it}x in {el:.1f} s (fp64 NumPy)",
               "gbs": total * it / el / 1e9, "affinity_cpus": len(os.sched_getaffinity(0)),
               "cpu_model": cpu_model()}
    achieved = total / (layer_us * 1e-6) / 1e9
    return {
        "value": rows * 1e3 / layer_ms, "unit": "rows/s", "ms_per_step": layer_ms,
        "steps": steps, "dtype": "bf16",
        "config": {"workload": f"decode_layer: {WORKLOAD_TEXT['decode_layer']}",
                   "path": "gather (projection sets)", "rows_per_step": rows,
                   "kernel_dispatches_per_step": 3, "rotating_copies": copies,
                   "timing": "HIP graphs of whole rotations over the copies plus the remainder, "
                             "replayed; HIP events on the replay stream"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic("decode_layer"),
                     "unit_of_work": "one decode layer: router fold, gate/up set, down fold",
                     "algorithmic_bytes": total, "algorithmic_bytes_per_fold": nbytes,
                     "step_us_mean": layer_us},
        "per_call": None if calls_us is None else {
            "four_calls_us": calls_us,
            "four_calls_frac": total / (calls_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "alone_us": alone,
            "alone_frac": {n: nbytes[n] / (alone[n] * 1e-6) / 1e9 / HBM_PEAK_GBS
                           for n in alone}},
        "cpu_baseline": cpu,
    }


def measure_multi(args, cpu_seconds):
    """The multi-adapter gather fold on the decode batch with four installed
    adapters (workloads.decode_multi_gather), timed as the other workloads
    are (graph replays over rotating copies of every input)."""
    import torch
    import moe_expert_lora_amd as ml
    import workloads
    from staging import DeviceMultiCase

    case = workloads.decode_multi_gather()
    copies = args.copies or max(2, min(64, math.ceil(640e6 / copy_bytes(case))))
    devs = [DeviceMultiCase(case) for _ in range(copies)]
    bases = [d.base0.clone() for d in devs]
    torch.cuda.synchronize()

    def step(k):
        d = devs[k]
        ml.mlora_gather_bgmv_multi(d.route, d.x, bases[k], d.indices, d.row_adapter,
                                   case.top_k)

    steps = args.steps
    rot = Rotation(step, copies, steps)
    rot.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    rot.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = e0.elapsed_time(e1) * 1e3 / steps
    # algorithmic bytes: cells and tokens of the folded rows, as for one adapter
    at, bt, st, na, ne = devs[0].tables_host
    ra = devs[0].row_adapter_host
    rows = np.arange(case.n_rows)
    tok = rows // case.top_k
    slot = ra[tok].astype(np.int64)
    e = case.indices.astype(np.int64)
    ok = (slot >= 0) & (slot < na) & (e >= 0) & (e < ne)
    cell = np.where(ok, slot * ne + e, 0)
    live = ok & (at[cell] != 0) & (bt[cell] != 0)
    K, N, R = case.k_in, case.n_out, case.max_rank
    nbytes = int(np.unique(tok[live]).size * K * 2 + np.unique(cell[live]).size *
                 (R * K + N * R) * 2 + live.sum() * N * 4 + 4 * case.n_rows + 4 * len(ra) +
                 20 * na * ne)
    del rot, devs, bases
    torch.cuda.empty_cache()
    cpu = None
    if cpu_seconds > 0:
        from oracle.case import OracleMultiView, to_f64
        from threadpoolctl import threadpool_limits
        import oracle
        v = OracleMultiView(case)
        b64 = to_f64(case.base, case.dtype)
        threads = cpu_threads()
        with threadpool_limits(limits=threads):
            v.fold(case.base)
            t1 = time.perf_counter()
            it = 0
            while True:
                oracle.fold_gather_multi(v.x, v.a_table, v.b_table, v.scale_table,
                                         v.n_adapters, v.n_experts, v.mats, b64, case.indices,
                                         v.row_adapter, case.top_k)
                it += 1
                el = time.perf_counter() - t1
                if (el >= cpu_seconds and it >= 3) or el >= 3 * cpu_seconds:
                    break
        cpu = {"value": case.n_rows * it / el, "unit": "rows/s", "cores": threads,
               "kind": "oracle", "sample": f"the full call, {it}x in {el:.1f} s (fp64, one "
                                           "row at a time)",
               "gbs": nbytes * it / el / 1e9, "affinity_cpus": len(os.sched_getaffinity(0)),
               "cpu_model": cpu_model()}
    achieved = nbytes / (step_us * 1e-6) / 1e9
    return {"value": case.n_rows * steps / wall, "unit": "rows/s",
            "ms_per_step": wall / steps * 1e3, "steps": steps, "dtype": "bf16",
            "config": {"workload": f"decode_multi_gather: {WORKLOAD_TEXT['decode_multi_gather']}",
                       "path": "gather (multi-adapter)", "rows_per_step": case.n_rows,
                       "folded_rows_per_step": int(live.sum()), "kernel_dispatches_per_step": 1,
                       "rotating_copies": copies},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                         "traffic": recorded_traffic("decode_multi_gather"),
                         "unit_of_work": "one mlora_gather_bgmv_multi call",
                         "algorithmic_bytes": nbytes, "step_us_mean": step_us},
            "cpu_baseline": cpu}


def resolve_workloads(workload, also):
    """(main workload, workloads reported under 'also') from the command line:
    no --workload means the decode default with every other measured workload
    beside it; an explicit --workload runs alone unless --also names others;
    --also none runs none."""
    if also is None:
        also = ",".join(w for w in MEASURED if w != DEFAULT_WORKLOAD) if workload is None else ""
    elif also == "none":
        also = ""
    workload = workload or DEFAULT_WORKLOAD
    extra = [w for w in also.split(",") if w and w != workload]
    for w in extra:
        if w not in WORKLOAD_TEXT:
            raise SystemExit(f"bench.py: unknown workload {w!r} in --also")
    return workload, extra


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOAD_TEXT),
                    help=f"default {DEFAULT_WORKLOAD}")
    ap.add_argument("--copies", type=int, default=0, help="rotating input copies (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the main one and reported "
                         "under 'also' (default: every other measured workload when no "
                         "--workload is given; 'none' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle budget of the main workload (each 'also' one: 60%%)")
    ap.add_argument("--one-kernel", action="store_true",
                    help="run the folds without a workspace (one-kernel forms)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of graph replays")
    ap.add_argument("--counters", action="store_true",
                    help="counter runs: warm-up and the timed steps only (cold inputs), no "
                         "CPU leg, no warm or spread passes")
    ap.add_argument("--floor-copy", action="store_true",
                    help="only time the plain-copy floor of the workload's algorithmic bytes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain copy used to scale HBM counters")
    ap.add_argument("--probes", action="store_true",
                    help="only run the launch and read-pattern probes (libmlora_probe.so)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc output dirs -> profiles/traffic.json (no GPU)")
    args = ap.parse_args()

    args.workload, args.also = resolve_workloads(args.workload, args.also)
    if args.traffic_from:
        traffic_from(args.workload, *args.traffic_from)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fold needs no collective and this "
              "build runs on a single MI355X. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("bench.py: --steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_expert_lora_amd as ml

    ml.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.probes:
        print(json.dumps({"probes": probes()}), flush=True)
        return
    if args.floor_copy:
        import workloads
        case = workloads.WORKLOADS[args.workload]()
        tables, ra = _tables_and_map(case)
        groups = (all_windows_groups(case.n_rows, case.cap)
                  if case.path == "grouped" and not args.one_kernel else None)
        n = algorithmic_traffic(case, tables, ra, groups)[0]
        us, gbs = copy_floor(n, args.steps)
        print(json.dumps({"workload": args.workload, "copy_bytes": n, "steps": args.steps,
                          "copy_us": us, "copy_gbs": gbs}), flush=True)
        return

    if args.counters:
        args.no_cpu = True
    main_cpu = 0.0 if args.no_cpu else args.cpu_seconds
    if args.workload in ("decode_layer", "decode_multi_gather"):
        if args.counters:
            # counter runs of these two: their own launches only
            fn = measure_layer if args.workload == "decode_layer" else measure_multi
            print(json.dumps({args.workload: fn(args, 0.0)}), flush=True)
            return
        print(f"bench.py: {args.workload} is reported under 'also' of another workload "
              f"(e.g. --workload decode_down_gather --also {args.workload})", file=sys.stderr)
        sys.exit(2)
    out = measure(args.workload, args, main_cpu)
    if not args.counters:
        out["hbm_copy_gbs"] = copy_bandwidth()
    # The metric covers the decode and the prefill halves of the fold: the
    # main line, and every other workload beside it, measured the same way.
    if args.also:
        out["also"] = {}
        for w in args.also:
            if w in ("decode_layer", "decode_multi_gather"):
                fn = measure_layer if w == "decode_layer" else measure_multi
                out["also"][w] = fn(args, 0.0 if args.no_cpu else 0.6 * args.cpu_seconds)
                continue
            r = measure(w, args, 0.0 if args.no_cpu else 0.6 * args.cpu_seconds)
            out["also"][w] = {k: r[k] for k in ("value", "unit", "ms_per_step", "steps",
                                                 "dtype", "config", "roofline",
                                                 "cpu_baseline") if k in r}
            for k in ("warm_step_us", "copy_floor", "eager_step_us", "host_loop_baseline"):
                if k in r:
                    out["also"][w][k] = r[k]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
