"""Oracle view of one seeded workload (test infrastructure only).

Turns a ``workloads.FoldCase`` (raw generator output: bf16 bit patterns,
packing entries naming weight handles, adapter slots, routing) into the fp64
inputs of the oracle folds, building the expert tables and the per-row adapter
map with the oracle's own host functions. Nothing here comes from the device
library.
"""
from __future__ import annotations

import numpy as np

from . import fold as _fold
from . import host as _host
from workloads import NULL_HANDLE, FoldCase


def oracle_addr(kind: str, handle: int) -> int:
    """Opaque, non-zero, distinct addresses for the oracle's tables (0 for the
    null handle, which marks an unadapted cell)."""
    if handle == NULL_HANDLE:
        return 0
    return 2 * (handle + 1) + (0 if kind == "a" else 1)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Generator storage (bf16 bits as uint16, or float32) to exact float64."""
    if dtype == "bf16":
        return _fold.bf16_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


class OracleView:
    """fp64 view of a FoldCase, with the tables and maps built by the oracle."""

    def __init__(self, case: FoldCase):
        self.case = case
        self.x = to_f64(case.x, case.dtype)
        self.entries = [(e, oracle_addr("a", a), oracle_addr("b", b), s)
                        for (e, a, b, s) in case.entries]
        packed = _host.pack_expert_tables(self.entries)
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
            self.row_adapter = np.asarray(_host.build_moe_row_adapter_decode(
                case.adapter_slots, case.padded_n, case.active, case.has_moe_lora),
                dtype=np.int32)
        else:
            m = _host.build_moe_row_adapter_host(case.cu_seqlens, case.stream_slots)
            assert m is not None
            self.row_adapter = np.asarray(m, dtype=np.int32)

    def windows(self):
        c = self.case
        return _host.grouped_down_windows(c.n_rows, c.cap)

    def _fold_with(self, x, mats, scales, base64, windows):
        c = self.case
        if c.path == "gather":
            # slot-major cases (notes["x_rows"] == "row") read x at the flat row
            return _fold.fold_gather(x, self.a_table, self.b_table, scales, mats, base64,
                                     c.indices, self.row_adapter, c.top_k,
                                     x_rows=c.notes.get("x_rows", "token"))
        if windows is None:
            windows = self.windows()
        return _fold.fold_grouped_windows(x, self.a_table, self.b_table, scales, mats, base64,
                                          c.expert_offsets, c.sorted_ids, self.row_adapter,
                                          c.top_k, windows)

    def fold(self, base=None, windows=None) -> np.ndarray:
        """The fp64, unrounded fold of the case on ``base`` (default: its own)."""
        c = self.case
        base64 = to_f64(c.base if base is None else base, c.dtype)
        return self._fold_with(self.x, self.mats, self.scale_table, base64, windows)

    def magnitude(self, windows=None) -> np.ndarray:
        """Per output element, |scale_e| * sum_j |B_e[n, j]| * sum_k |A_e[j, k]| |x[t, k]|
        (0 on rows that fold nothing): the sum of the absolute values of every
        product that enters the element's delta, which scales the rounding
        error of any evaluation of the delta in floating point."""
        c = self.case
        mats = {k: np.abs(m) for k, m in self.mats.items()}
        scales = [abs(float(s)) for s in self.scale_table]
        zero = np.zeros(c.base.shape, dtype=np.float64)
        return self._fold_with(np.abs(self.x), mats, scales, zero, windows)

    def live_rows(self) -> np.ndarray:
        """Boolean mask of rows that the fold writes: the skip rules of the
        oracle folds, row by row."""
        c = self.case
        n = self.n_experts

        def cell(e):
            return 0 <= e < n and self.a_table[e] != 0 and self.b_table[e] != 0

        live = np.zeros(c.n_rows, dtype=bool)
        if c.path == "gather":
            for row in range(c.n_rows):
                live[row] = (self.row_adapter[row // c.top_k] >= 0) and cell(int(c.indices[row]))
            return live
        off = c.expert_offsets
        n_tok = self.x.shape[0]
        for e in range(len(off) - 1):
            if not cell(e):
                continue
            for r in range(max(int(off[e]), 0), min(int(off[e + 1]), c.n_rows)):
                rid = int(c.sorted_ids[r])
                if rid < 0 or rid // c.top_k >= n_tok:
                    continue
                live[r] = self.row_adapter[rid // c.top_k] >= 0
        return live


class OracleMultiView:
    """fp64 view of a multi-adapter FoldCase (workloads.make_multi_gather_case):
    tables packed and the map built by the oracle's multi-adapter functions."""

    def __init__(self, case: FoldCase):
        from . import multi as _multi
        self.case = case
        self.x = to_f64(case.x, case.dtype)
        self.entries = [(sl, e, oracle_addr("a", a), oracle_addr("b", b), s)
                        for (sl, e, a, b, s) in case.notes["multi_entries"]]
        (self.a_table, self.b_table, self.scale_table, self.n_adapters,
         self.n_experts) = _multi.pack_expert_tables_multi(self.entries)
        self.mats = {}
        for (_, _, a, b, _) in case.notes["multi_entries"]:
            self.mats[oracle_addr("a", a)] = to_f64(case.a_pool[a], case.dtype)
            self.mats[oracle_addr("b", b)] = to_f64(case.b_pool[b], case.dtype)
        self.row_adapter = np.asarray(_multi.build_moe_row_adapter_decode_multi(
            case.adapter_slots, case.padded_n, case.notes["n_adapters"]), dtype=np.int32)

    def fold(self, base=None) -> np.ndarray:
        from . import multi as _multi
        c = self.case
        base64 = to_f64(c.base if base is None else base, c.dtype)
        return _multi.fold_gather_multi(self.x, self.a_table, self.b_table, self.scale_table,
                                        self.n_adapters, self.n_experts, self.mats, base64,
                                        c.indices, self.row_adapter, c.top_k)

    def magnitude(self) -> np.ndarray:
        from . import multi as _multi
        c = self.case
        mats = {k: np.abs(m) for k, m in self.mats.items()}
        return _multi.fold_gather_multi(np.abs(self.x), self.a_table, self.b_table,
                                        [abs(float(v)) for v in self.scale_table],
                                        self.n_adapters, self.n_experts, mats,
                                        np.zeros(c.base.shape), c.indices, self.row_adapter,
                                        c.top_k)

    def live_rows(self) -> np.ndarray:
        c = self.case
        live = np.zeros(c.n_rows, dtype=bool)
        for row in range(c.n_rows):
            sl = int(self.row_adapter[row // c.top_k])
            e = int(c.indices[row])
            if 0 <= sl < self.n_adapters and 0 <= e < self.n_experts:
                cell = sl * self.n_experts + e
                live[row] = self.a_table[cell] != 0 and self.b_table[cell] != 0
        return live

