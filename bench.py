"""Benchmark of the MoE expert-LoRA fold on one MI355X.

One step = one pass of the fold over one synthetic batch: for the decode
workloads one mlora_gather_bgmv call, for the prefill workloads one
mlora_grouped_down call per window of grouped_down_windows. The host-side
integer work (tables, maps, windows) is done once before timing, as an engine
does at adapter install / batch setup; its cost is reported separately.
Steps are captured in a HIP graph and replayed (the fold reads its routing on
the device precisely so that it can be captured); eager launch cost, which
the host launch path dominates for the small decode calls, is reported too.

Inputs are resident in HBM before timing starts. The step cycles through
`copies` independent copies of x, A, B, base_out and the tables, so each step
reads data that no recent step touched (more bytes than L2 + MALL hold):
the figures are cold-cache HBM figures.

Prints ONE JSON line (rank 0, N = 1):
  value      rows folded per second (rows covered by the calls / wall time)
  roofline   algorithmic bytes per launch / mean launch duration (HIP events)
             against the 8 TB/s HBM peak; traffic = counter-measured HBM bytes
             from the committed rocprofv3 summary when the kernel source still
             matches it, else null
  cpu_baseline  the fp64 CPU oracle timed on the host on a bounded sample
  also       (default run) the prefill grouped workload measured the same way:
             value, ms_per_step, config and roofline of its own
  warm_launch_us  the same call replayed on one copy, inputs resident in L2 /
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
KERNEL_SOURCE = os.path.join(ROOT, "moe_expert_lora_amd", "csrc", "mlora_fold.hip")
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
}


def kernel_hash() -> str:
    """Hash of the kernel source's code: line comments and blank lines are
    dropped first, so an edit of the comments keeps recorded counters valid."""
    code = []
    with open(KERNEL_SOURCE) as f:
        for line in f:
            line = line.split("//", 1)[0].rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes: what the fold must move, counted from the inputs
# ---------------------------------------------------------------------------

def algorithmic_traffic(case, tables, row_adapter):
    """(bytes, flops, rows, folded_rows) per step, summed over launches.

    bytes = unique tokens * k_in * 2 + unique experts * (r*k_in + n_out*r) * 2
          + folded rows * n_out * 2 * 2 (base_out read + write)
          + 4 * rows (indices / sorted_ids) + 4 * tokens (map)
          + 4 * (n_route + 1) (offsets, grouped) + 20 * n_experts (tables)
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

    launches = []
    if case.path == "gather":
        rows = np.arange(case.n_rows)
        tok = rows // case.top_k
        e = case.indices.astype(np.int64)
        live = (ra[tok] >= 0) & cell_ok(e)
        launches.append((case.n_rows, tok[live], e[live], 0))
    else:
        off = case.expert_offsets.astype(np.int64)
        owner = np.searchsorted(off, np.arange(case.n_rows), side="right") - 1
        tok_all = case.sorted_ids.astype(np.int64) // case.top_k
        inside = (owner >= 0) & (owner < len(off) - 1)
        import moe_expert_lora_amd as ml
        for (s, t) in ml.mlora_grouped_down_windows(case.n_rows, case.cap):
            o = owner[s:t]
            tk = tok_all[s:t]
            live = inside[s:t] & cell_ok(o) & (ra[np.clip(tk, 0, len(ra) - 1)] >= 0)
            launches.append((t - s, tk[live], o[live], case.n_route + 1))
    total_b = 0
    flops = 0
    folded = 0
    rows_total = 0
    for (rows, toks, exps, n_off) in launches:
        f = toks.shape[0]
        b = (np.unique(toks).size * K * elt + np.unique(exps).size * (R * K + N * R) * elt
             + f * N * elt * 2 + 4 * rows + 4 * case.n_tokens + 4 * n_off + 20 * n_exp)
        total_b += int(b)
        flops += 2 * f * R * (K + N)
        folded += f
        rows_total += rows
    return total_b, flops, rows_total, folded, len(launches)


# ---------------------------------------------------------------------------
# device staging with rotating copies
# ---------------------------------------------------------------------------

class Staged:
    def __init__(self, case, copies, device="cuda", two_kernel=True):
        import torch
        from tests.device import DeviceCase
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
        from tests.device import u64_to_device
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

def cpu_baseline(case, budget_s=10.0):
    from tests.common import OracleView
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    view = OracleView(case)
    base64 = None
    from tests.common import to_f64
    base64 = to_f64(case.base, case.dtype)
    import oracle

    if case.path == "gather":
        def run():
            return oracle.fold_gather(view.x, view.a_table, view.b_table, view.scale_table,
                                      view.mats, base64, case.indices, view.row_adapter,
                                      case.top_k)
        rows_per = case.n_rows
        sample = f"full {case.name} fold ({rows_per} rows) repeated"
    else:
        # bounded sample: the first window
        import moe_expert_lora_amd as ml
        s, e = ml.mlora_grouped_down_windows(case.n_rows, case.cap)[0]

        def run():
            return oracle.fold_grouped(view.x, view.a_table, view.b_table, view.scale_table,
                                       view.mats, base64, case.expert_offsets, case.sorted_ids,
                                       view.row_adapter, case.top_k, s, e)
        rows_per = e - s
        sample = f"first window [{s}, {e}) of {case.name}, repeated"
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
            "kind": "oracle", "sample": f"{sample} {iters}x in {el:.1f} s (fp64 NumPy, "
                                         "per-expert matmuls)"}


# ---------------------------------------------------------------------------


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


def traffic_from(workload, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir):
    """Per-launch HBM bytes of the fold from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the counter reads for the plain copy of
    CALIB_BYTES; recorded in profiles/traffic.json with the kernel hash.

    A step is one or more fold kernels (a shrink and an expand; the pipelined
    grouped call adds one launch per later group of windows). Every kernel runs at least
    once per step, so the least frequent one counts the steps, and the
    per-launch figure is the counters summed over all fold dispatches divided
    by steps x launches per step (windows, for grouped workloads)."""
    is_copy = lambda n: "mlora" not in n  # noqa: E731
    rows_f, rows_w = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    names = sorted({r["Kernel_Name"] for r in rows_f + rows_w if "mlora" in r["Kernel_Name"]})
    import workloads
    case = workloads.WORKLOADS[workload]()
    launches = algorithmic_traffic(case, *_tables_and_map(case))[4]

    def per_launch(rows, counter):
        vals = {n: [float(r["Counter_Value"]) for r in rows
                    if r["Counter_Name"] == counter and r["Kernel_Name"] == n] for n in names}
        steps = min(len(v) for v in vals.values())
        total = sum(sum(v) for v in vals.values())
        return total / (steps * launches), [len(v) for v in vals.values()]

    f_kib, nf = per_launch(rows_f, "FETCH_SIZE")
    w_kib, nw = per_launch(rows_w, "WRITE_SIZE")
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
        "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
        "kernels": [re.sub(r"(?<=>)\(.*$", "", n.replace("void mlora::(anonymous namespace)::", ""))
                    for n in names],
        "dispatches": [nf, nw],
        "launches_per_step": launches,
        "copy_scale_fetch": kf, "copy_scale_write": kw,
        "hbm_bytes_per_launch": f_kib * 1024.0 * kf + w_kib * 1024.0 * kw,
    }
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[workload] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({workload: rec}))


def measure(workload, args, with_cpu):
    """One workload: stage it, time `args.steps` graph-replayed steps, and
    return the result record (the JSON line's fields)."""
    import torch
    import moe_expert_lora_amd as ml
    import workloads

    case = workloads.WORKLOADS[workload]()
    cb = copy_bytes(case)
    copies = args.copies or max(2, min(64, math.ceil(640e6 / cb)))
    st = Staged(case, copies, two_kernel=not args.one_kernel)
    tables = st.primary.tables_host
    ra = st.primary.row_adapter_host
    alg_bytes, flops, rows, folded, launches = algorithmic_traffic(case, tables, ra)

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

    # The fold reads its routing on the device, so a step is captured once in a
    # HIP graph and replayed, as a decode loop runs it. One graph holds one step
    # per rotating copy; K steps are K / copies replays (K rounded up).
    for i in range(args.warmup):
        st.step(i)
    torch.cuda.synchronize()
    if args.eager:
        class _Eager:
            def replay(self):
                for i in range(copies):
                    st.step(i)
        graph = _Eager()
    else:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for i in range(copies):
                    st.step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
    replays = max(1, math.ceil(args.steps / copies))
    steps = replays * copies
    for _ in range(max(1, math.ceil(args.warmup / copies))):
        graph.replay()
    torch.cuda.synchronize()

    # timed region: `steps` steps, wall clock and HIP events on the replay stream
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_replay = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(replays):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / steps
    per_launch_s = step_ms / 1e3 / launches

    # spread of the per-replay duration (a second, separately timed pass)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for r in range(replays):
        ev[r][0].record(stream)
        graph.replay()
        ev[r][1].record(stream)
    torch.cuda.synchronize()
    dur_ms = np.array([a.elapsed_time(b) for a, b in ev]) / copies

    # eager launches (host launch path included), for the record
    t0 = time.perf_counter()
    for i in range(copies):
        st.step(i)
    torch.cuda.synchronize()
    eager_us = (time.perf_counter() - t0) / copies * 1e6

    # warm figure, for context: one copy's step, captured as many times as the
    # cold graph holds steps (the same graph-launch cost per step) and
    # replayed, its inputs resident in L2 / MALL after the first step
    warm_us = None
    if not args.eager:
        wg = torch.cuda.CUDAGraph()
        side2 = torch.cuda.Stream()
        side2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side2):
            with torch.cuda.graph(wg, stream=side2):
                for _ in range(copies):
                    st.step(0)
        torch.cuda.current_stream().wait_stream(side2)
        wg.replay()
        torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for _ in range(replays):
            wg.replay()
        w1.record(stream)
        torch.cuda.synchronize()
        warm_us = w0.elapsed_time(w1) * 1e3 / (replays * copies) / launches

    achieved = alg_bytes / launches / per_launch_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            rec = json.load(open(TRAFFIC_FILE)).get(workload)
            if rec and rec.get("kernel_sha256_16") == kernel_hash():
                traffic = rec.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    cpu = None
    if with_cpu:
        cpu = cpu_baseline(case, args.cpu_seconds)

    ms_per_step = wall / steps * 1e3
    out = {
        "metric": METRIC,
        "value": rows * steps / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
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
            "launches_per_step": launches,
            "workspace": not args.one_kernel,
            "rotating_copies": copies,
            "timing": ("eager launches" if args.eager else
                       "HIP graph of one step per copy, replayed"),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes / launches,
            "flops_per_launch": flops / launches,
            "launch_us_mean": per_launch_s * 1e6,
            "step_us_p10_p50_p90": [float(np.percentile(dur_ms, q)) * 1e3 for q in (10, 50, 90)],
        },
        "cpu_baseline": cpu,
        "host_setup_us": host_us,
        "eager_step_us": eager_us,
        "warm_launch_us": warm_us,
        "notes": "the pages quote no performance numbers; vs_baseline is null",
    }
    return out


def resolve_workloads(workload, also):
    """(main workload, workloads reported under 'also') from the command line:
    no --workload means the decode default with the prefill grouped workload
    beside it; an explicit --workload runs alone unless --also names others;
    --also none runs none."""
    if also is None:
        also = "prefill_grouped_down" if workload is None else ""
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
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the main one and reported "
                         "under 'also' (default: the prefill grouped workload when no "
                         "--workload is given; 'none' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--one-kernel", action="store_true",
                    help="run the folds without a workspace (one-kernel forms)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of graph replays")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the plain copy used to scale HBM counters")
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

    import torch
    import moe_expert_lora_amd as ml

    ml.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return

    out = measure(args.workload, args, with_cpu=not args.no_cpu)
    out["hbm_copy_gbs"] = copy_bandwidth()
    # The metric covers both halves of the fold: the decode line above, and
    # the prefill grouped workload beside it (same protocol, no CPU leg).
    also = args.also
    if also:
        out["also"] = {}
        for w in also:
            r = measure(w, args, with_cpu=False)
            out["also"][w] = {k: r[k] for k in ("value", "unit", "ms_per_step", "steps",
                                                 "dtype", "config", "roofline")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
