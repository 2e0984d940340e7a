"""fp64 oracle of the two fold entry points.

Both restate the fold of the "moe_lora_grouped" index page: each live row
``row`` gets ``base_out[row] + scale_e * ((x[token] @ A_e^T) @ B_e^T)``,

* gather (item ``moe_lora_gather_bgmv``): rows are the flat ``(token, slot)``
  decode rows, ``token = row // top_k`` (item ``gather_row_token``), and the
  expert is ``indices[row]``;
* grouped (item ``moe_lora_grouped_down``): rows are expert-sorted prefill rows
  inside the window ``[row_offset, row_end)``; the expert is the one whose
  half-open ``expert_offsets`` span holds the row, and the token is
  ``sorted_ids[row] // top_k`` (a reading: the sorted row keeps its flat
  ``(token, slot)`` id).

A row folds nothing (it is returned exactly as given) when

* its token's adapter map entry is negative ("moe_row_adapter.rs", the module
  doc and ``build_moe_row_adapter_decode``),
* its expert id is negative or at/after the table length, or the expert's
  ``a_table`` or ``b_table`` cell is 0 (the invariant on the "moe_lora_grouped"
  index page),
* (grouped) it lies in no span, or outside the window, or its sorted id does
  not name a token of ``x``: a negative id (a padding row of the router's
  sorted output) or an id whose token ``id // top_k`` is at/after the last
  row of ``x``. The pages do not name the sorted-row map; reading it as the
  flat ``(token, slot)`` id, an id that names no token has no ``x`` row to
  fold, so the row is left as given.

Shapes (a reading stated with the route fields ``k_in``, ``n_out``,
``max_rank``): ``x [n_tokens, k_in]``, ``A_e [max_rank, k_in]``,
``B_e [n_out, max_rank]``, ``base [n_rows, n_out]``. ``mats`` maps a table
address to its matrix (fp64). Results are fp64 and unrounded.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64: a bf16 value is the fp32 value
    whose upper 16 bits are the pattern and lower 16 bits are zero."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _cell_live(e: int, a_table, b_table) -> bool:
    n = len(a_table)
    if e < 0 or e >= n:
        return False
    return a_table[e] != 0 and b_table[e] != 0


def fold_gather_scalar(x: np.ndarray, a_table: Sequence[int], b_table: Sequence[int],
                       scale_table: Sequence[float], mats: Dict[int, np.ndarray],
                       base: np.ndarray, indices: Sequence[int], row_adapter: Sequence[int],
                       top_k: int, x_rows: str = "token") -> np.ndarray:
    """Gather fold, one row at a time. ``x_rows`` says which x row a flat row
    reads: "token" (x[row // top_k], token-major x, the page's x[token(row)])
    or "row" (x[row], slot-major x with one row per (token, slot) row, the
    page's x[x_row] read as the down projection's per-slot input). The
    adapter map is indexed by the token either way."""
    out = np.array(base, dtype=np.float64, copy=True)
    for row in range(len(indices)):
        t = row // top_k
        if row_adapter[t] < 0:
            continue
        e = int(indices[row])
        if not _cell_live(e, a_table, b_table):
            continue
        a = mats[a_table[e]]
        b = mats[b_table[e]]
        xr = x[t] if x_rows == "token" else x[row]
        h = a @ xr                         # [max_rank]
        delta = float(scale_table[e]) * (b @ h)  # [n_out]
        out[row] = base[row] + delta
    return out


def fold_gather(x: np.ndarray, a_table, b_table, scale_table, mats, base: np.ndarray,
                indices, row_adapter, top_k: int, x_rows: str = "token") -> np.ndarray:
    """Gather fold, one expert at a time: the live rows of each packed expert
    are gathered and folded with two matrix products. ``x_rows`` as for
    :func:`fold_gather_scalar`."""
    if x_rows not in ("token", "row"):
        raise ValueError(x_rows)
    out = np.array(base, dtype=np.float64, copy=True)
    indices = np.asarray(indices, dtype=np.int64)
    row_adapter = np.asarray(row_adapter, dtype=np.int64)
    n_slots = indices.shape[0]
    rows = np.arange(n_slots)
    tok = rows // top_k
    live = row_adapter[tok] >= 0 if n_slots else np.zeros(0, dtype=bool)
    for e in range(len(a_table)):
        if not _cell_live(e, a_table, b_table):
            continue
        sel = rows[live & (indices == e)]
        if sel.size == 0:
            continue
        a = mats[a_table[e]]
        b = mats[b_table[e]]
        xs = x[tok[sel]] if x_rows == "token" else x[sel]
        h = xs @ a.T                       # [m, max_rank]
        out[sel] = base[sel] + float(scale_table[e]) * (h @ b.T)
    return out


def _owner(r: int, offsets: Sequence[int]) -> int:
    for e in range(len(offsets) - 1):
        if offsets[e] <= r < offsets[e + 1]:
            return e
    return -1


def _sorted_token(row_id: int, top_k: int, n_tokens: int) -> int:
    """Token of a sorted row's flat ``(token, slot)`` id, or -1 when the id
    names no row of ``x`` (negative, or its token is ``n_tokens`` or more)."""
    if row_id < 0:
        return -1
    t = row_id // top_k
    return t if t < n_tokens else -1


def fold_grouped_scalar(x: np.ndarray, a_table, b_table, scale_table, mats,
                        base: np.ndarray, expert_offsets, sorted_ids, row_adapter,
                        top_k: int, row_offset: int, row_end: int) -> np.ndarray:
    """Grouped fold over the window ``[row_offset, row_end)``, one row at a time."""
    out = np.array(base, dtype=np.float64, copy=True)
    offsets = [int(v) for v in expert_offsets]
    for r in range(row_offset, row_end):
        e = _owner(r, offsets)
        if e < 0:
            continue
        t = _sorted_token(int(sorted_ids[r]), top_k, x.shape[0])
        if t < 0:
            continue
        if row_adapter[t] < 0:
            continue
        if not _cell_live(e, a_table, b_table):
            continue
        a = mats[a_table[e]]
        b = mats[b_table[e]]
        out[r] = base[r] + float(scale_table[e]) * (b @ (a @ x[t]))
    return out


def fold_grouped(x: np.ndarray, a_table, b_table, scale_table, mats, base: np.ndarray,
                 expert_offsets, sorted_ids, row_adapter, top_k: int, row_offset: int,
                 row_end: int) -> np.ndarray:
    """Grouped fold over one window, one expert span at a time."""
    out = np.array(base, dtype=np.float64, copy=True)
    offsets = np.asarray(expert_offsets, dtype=np.int64)
    sorted_ids = np.asarray(sorted_ids, dtype=np.int64)
    row_adapter = np.asarray(row_adapter, dtype=np.int64)
    for e in range(offsets.shape[0] - 1):
        lo = max(int(offsets[e]), row_offset)
        hi = min(int(offsets[e + 1]), row_end)
        if hi <= lo:
            continue
        if not _cell_live(e, a_table, b_table):
            continue
        rows = np.arange(lo, hi)
        ids = sorted_ids[rows]
        named = (ids >= 0) & (ids // top_k < x.shape[0])
        rows, tok = rows[named], ids[named] // top_k
        keep = row_adapter[tok] >= 0
        rows, tok = rows[keep], tok[keep]
        if rows.size == 0:
            continue
        a = mats[a_table[e]]
        b = mats[b_table[e]]
        out[rows] = base[rows] + float(scale_table[e]) * ((x[tok] @ a.T) @ b.T)
    return out


def fold_grouped_windows(x, a_table, b_table, scale_table, mats, base, expert_offsets,
                         sorted_ids, row_adapter, top_k, windows) -> np.ndarray:
    """Apply :func:`fold_grouped` window after window (each on the previous
    result), as a caller that splits the rows does."""
    out = np.array(base, dtype=np.float64, copy=True)
    for (s, e) in windows:
        out = fold_grouped(x, a_table, b_table, scale_table, mats, out, expert_offsets,
                           sorted_ids, row_adapter, top_k, s, e)
    return out
