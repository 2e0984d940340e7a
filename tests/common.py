"""Shared test helpers: turn a seeded FoldCase into oracle inputs and results,
and the parity metrics used by every fold comparison."""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from workloads import NULL_HANDLE, FoldCase

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerance for the bf16-in / fp32-accumulate fold against the fp64 oracle.
REL_L2_TOL = 2e-3
MAX_ABS_TOL = 3e-2


def golden_lines(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def golden_json(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def oracle_addr(kind: str, handle: int) -> int:
    """Opaque, non-zero, distinct addresses for the oracle's tables."""
    if handle == NULL_HANDLE:
        return 0
    return 2 * (handle + 1) + (0 if kind == "a" else 1)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return oracle.bf16_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


class OracleView:
    """fp64 view of a FoldCase, with the tables and maps built by the oracle."""

    def __init__(self, case: FoldCase):
        self.case = case
        self.x = to_f64(case.x, case.dtype)
        self.entries = [(e, oracle_addr("a", a), oracle_addr("b", b), s)
                        for (e, a, b, s) in case.entries]
        packed = oracle.pack_expert_tables(self.entries)
        if packed is None:
            self.a_table, self.b_table, self.scale_table, self.n_experts = [], [], [], 0
        else:
            self.a_table, self.b_table, self.scale_table, self.n_experts = packed
        self.mats = {}
        handles = {a for (_, a, _, _) in case.entries} | {b for (_, _, b, _) in case.entries}
        for h in handles:
            if h == NULL_HANDLE:
                continue
            self.mats[oracle_addr("a", h)] = to_f64(case.a_pool[h], case.dtype)
            self.mats[oracle_addr("b", h)] = to_f64(case.b_pool[h], case.dtype)
        if case.map_kind == "decode":
            self.row_adapter = np.asarray(oracle.build_moe_row_adapter_decode(
                case.adapter_slots, case.padded_n, case.active, case.has_moe_lora),
                dtype=np.int32)
        else:
            m = oracle.build_moe_row_adapter_host(case.cu_seqlens, case.stream_slots)
            assert m is not None
            self.row_adapter = np.asarray(m, dtype=np.int32)

    def fold(self, base=None, windows=None) -> np.ndarray:
        c = self.case
        base64 = to_f64(c.base if base is None else base, c.dtype)
        if c.path == "gather":
            return oracle.fold_gather(self.x, self.a_table, self.b_table, self.scale_table,
                                      self.mats, base64, c.indices, self.row_adapter, c.top_k)
        if windows is None:
            windows = oracle.grouped_down_windows(c.n_rows, c.cap)
        return oracle.fold_grouped_windows(self.x, self.a_table, self.b_table,
                                           self.scale_table, self.mats, base64,
                                           c.expert_offsets, c.sorted_ids, self.row_adapter,
                                           c.top_k, windows)

    def live_rows(self) -> np.ndarray:
        """Boolean mask of rows that the fold writes."""
        c = self.case
        n = self.n_experts

        def cell(e):
            return 0 <= e < n and self.a_table[e] != 0 and self.b_table[e] != 0

        live = np.zeros(c.n_rows, dtype=bool)
        if c.path == "gather":
            for row in range(c.n_rows):
                live[row] = (self.row_adapter[row // c.top_k] >= 0) and cell(int(c.indices[row]))
        else:
            off = c.expert_offsets
            for e in range(len(off) - 1):
                if not cell(e):
                    continue
                for r in range(int(off[e]), int(off[e + 1])):
                    if 0 <= r < c.n_rows:
                        live[r] = self.row_adapter[int(c.sorted_ids[r]) // c.top_k] >= 0
        return live


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(got - ref))
    return num / den if den > 0 else num


def max_abs(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


def ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output format at |ref| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.abs(ref))  # |ref| = m * 2**e, m in [0.5, 1)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - bits)


def max_abs_excess(got: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    """Largest ratio |got - ref| / max(MAX_ABS_TOL, ulp(ref)); <= 1 passes.

    Reading of the max-abs bound: a value stored in bf16 can be off from the
    exact result by half an ulp, which exceeds 3e-2 once |value| >= 8, so the
    bound allows one output ulp where that is larger than 3e-2."""
    if not got.size:
        return 0.0
    lim = np.maximum(MAX_ABS_TOL, ulp(ref, dtype))
    return float(np.max(np.abs(got - ref) / lim))
