"""Oracle for the host-side integer work around the fold.

Each function restates one item of the pages in plain Python. Cited items:

* "moe_row_adapter.rs", items ``resolve_moe_lora_route``,
  ``ensure_decode_route_servable``, ``build_moe_row_adapter_host``,
  ``build_moe_row_adapter_decode`` (full source shown on that page);
* "moe_lora_grouped" module index, items ``pack_expert_tables``,
  ``ExpertTables``, ``grouped_down_windows``, ``grouped_down_wc``,
  ``gather_row_token``, ``MLG_M_TILE``.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

FOLD = "Fold"
SKIP = "Skip"
REFUSE = "Refuse"

# Reading of the pages (they use unsigned ids and never bound them): a packed
# expert id must lie in [0, 2**24) so the dense table stays modest.
MAX_EXPERT_ID = (1 << 24) - 1


class RefuseError(RuntimeError):
    """A decode batch holds a request for an adapter other than the active one."""


def resolve_moe_lora_route(adapter_slot: int, active: int, has_moe_lora: bool) -> str:
    """The fold decision for one request ("moe_row_adapter.rs",
    ``resolve_moe_lora_route``): no MoE LoRA loaded means Fold; a base request
    (negative slot) is Skip; the active slot is Fold; any other slot is Refuse,
    since only the active adapter's tables are installed."""
    if not has_moe_lora:
        return FOLD
    if adapter_slot < 0:
        return SKIP
    if adapter_slot == active:
        return FOLD
    return REFUSE


def ensure_decode_route_servable(route: str, path: str = "decode") -> None:
    """Raise when ``route`` is Refuse ("moe_row_adapter.rs",
    ``ensure_decode_route_servable``): a batch mixing adapters cannot be served
    by the single-active fold and must be rejected before it runs."""
    if route == REFUSE:
        raise RefuseError(f"MoE LoRA {path} refused: a request names an adapter whose "
                          "tables are not installed; serve it in a batch of its own")


def build_moe_row_adapter_host(cu_seqlens: Sequence[int],
                               adapter_slots: Sequence[int]) -> Optional[List[int]]:
    """Per-token adapter map of a packed prefill batch ("moe_row_adapter.rs",
    ``build_moe_row_adapter_host``).

    ``cu_seqlens`` are the stream boundaries, a prefix sum starting at 0
    (``batch + 1`` entries), and stream ``b`` owns tokens ``cu[b] .. cu[b+1]``;
    its slot is copied as is onto them. The input is valid when there are at
    least two boundaries, one slot per stream, the first boundary is 0 and no
    boundary is below the one before it (so none is negative); otherwise the
    result is None and nothing is built (so ``[0, 4, 2]`` is rejected rather
    than sized from its last entry).
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
    slots = np.asarray(adapter_slots, dtype=np.int64).reshape(-1)
    valid = (cu.size >= 2 and slots.size == cu.size - 1 and cu[0] == 0
             and bool(np.all(np.diff(cu) >= 0)))
    if not valid:
        return None
    return np.repeat(slots, np.diff(cu)).astype(int).tolist()


def build_moe_row_adapter_decode(adapter_slots: Sequence[int], padded_n: int, active: int,
                                 has_moe_lora: bool) -> List[int]:
    """Per-sequence adapter map of a decode batch ("moe_row_adapter.rs",
    ``build_moe_row_adapter_decode``): entry ``i`` (for ``i < padded_n``) is
    ``active`` when sequence ``i`` exists and its route is Fold, else -1; Skip,
    Refuse and padding entries are all -1. A slot list longer than
    ``padded_n`` is cut at ``padded_n``."""
    out = []
    for i in range(int(padded_n)):
        if i < len(adapter_slots):
            route = resolve_moe_lora_route(int(adapter_slots[i]), active, has_moe_lora)
            out.append(int(active) if route == FOLD else -1)
        else:
            out.append(-1)
    return out


def pack_expert_tables(entries: Sequence[Tuple[int, int, int, float]]):
    """Dense per-expert tables ("moe_lora_grouped" index, ``pack_expert_tables``
    and ``ExpertTables``).

    Entries are ``(expert_id, a_addr, b_addr, scale)``. The tables are indexed
    by expert id and have ``max id + 1`` cells; an id that no entry names gets
    a 0 address and scale 0.0; when an id repeats, the entry listed last
    wins. An empty list gives None. Ids outside ``[0, MAX_EXPERT_ID]`` raise
    ValueError (a reading: the pages use unsigned ids).

    Returns ``(a_table, b_table, scale_table, n_experts)`` with Python ints for
    the addresses and the scales as given.
    """
    if len(entries) == 0:
        return None
    for e, _, _, _ in entries:
        if not (0 <= int(e) <= MAX_EXPERT_ID):
            raise ValueError(f"expert id {e} out of range")
    n = max(int(e) for e, _, _, _ in entries) + 1
    a = [0] * n
    b = [0] * n
    s = [0.0] * n
    for e, aa, bb, sc in entries:
        a[int(e)] = int(aa)
        b[int(e)] = int(bb)
        s[int(e)] = sc
    return a, b, s, n


def grouped_down_windows(total_rows: int, cap: int) -> List[Tuple[int, int]]:
    """Contiguous ``[start, end)`` windows of at most ``cap`` rows that cover
    ``0 .. total_rows`` ("moe_lora_grouped" index, ``grouped_down_windows``).
    Reading: windows are filled greedily (all full except the last), zero rows
    give no window, and ``cap`` of 0 (the pages panic) raises ValueError."""
    if cap <= 0:
        raise ValueError("cap must be positive")
    if total_rows < 0:
        raise ValueError("total_rows must be non-negative")
    out = []
    start = 0
    while start < total_rows:
        end = min(start + cap, total_rows)
        out.append((start, end))
        start = end
    return out


def grouped_down_wc(row_offset: int, row_end: int, m_tile: int) -> int:
    """Row-tile count of one window ("moe_lora_grouped" index,
    ``grouped_down_wc``): the ceiling of the window length over the tile rows,
    never below 1."""
    length = row_end - row_offset
    tiles = -(-length // m_tile)  # ceiling division
    return max(1, tiles)


def gather_row_token(row: int, top_k: int) -> int:
    """The token that owns flat ``(token, slot)`` row ``row`` ("moe_lora_grouped"
    index, ``gather_row_token``): rows are token-major with ``top_k`` slots
    per token, so the token is the integer quotient."""
    return row // top_k
