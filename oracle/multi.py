"""Oracle of the multi-adapter gather fold (test infrastructure only).

The pages describe a single-active ("phase-1") design: only the active
adapter's expert tables are installed, the per-row map holds the active slot
or -1, and a decode batch that asks for any other adapter is refused
("moe_row_adapter.rs", items resolve_moe_lora_route and
ensure_decode_route_servable, which names the one-adapter-per-batch rule).
Lifting that refusal is read here as the plain generalisation of the same
rules (a reading; the pages stop at phase 1):

* every installed adapter slot has its own expert tables, packed as with
  pack_expert_tables ("moe_lora_grouped" index), into one table of
  n_adapters x n_experts cells indexed [slot][expert id];
* a request's route is Skip for a negative slot, Fold for a slot that has
  tables, and Refuse for a slot past them (the multi-adapter form of asking
  for an adapter that is not installed);
* the decode map keeps each folding request's own slot (-1 otherwise), and
  a row folds with the cell [row_adapter[token]][indices[row]], skipped as
  the single-adapter fold skips (negative map, id outside the table, a null
  cell) and also when the map names a slot past the tables.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

from .host import FOLD, REFUSE, SKIP, MAX_EXPERT_ID

MAX_ADAPTER_SLOT = (1 << 16) - 1  # a reading: slots are small integers


def resolve_moe_lora_route_multi(adapter_slot: int, n_adapters: int) -> str:
    """Skip for a negative slot, Fold for a slot with installed tables, Refuse
    for a slot past them."""
    if adapter_slot < 0:
        return SKIP
    if adapter_slot < n_adapters:
        return FOLD
    return REFUSE


def build_moe_row_adapter_decode_multi(adapter_slots: Sequence[int], padded_n: int,
                                       n_adapters: int) -> List[int]:
    """Per-sequence map of a decode batch: entry i (i < padded_n) is the
    sequence's own slot when its route is Fold, else -1 (Skip, Refuse,
    padding); a slot list longer than padded_n is cut at padded_n."""
    out = []
    for i in range(int(padded_n)):
        if i < len(adapter_slots):
            s = int(adapter_slots[i])
            out.append(s if resolve_moe_lora_route_multi(s, n_adapters) == FOLD else -1)
        else:
            out.append(-1)
    return out


def pack_expert_tables_multi(entries: Sequence[Tuple[int, int, int, int, float]]):
    """Entries (adapter_slot, expert_id, a_addr, b_addr, scale) into dense
    tables of n_adapters x n_experts cells, cell (s, e) at s * n_experts + e,
    with n_adapters = max slot + 1 and n_experts = max id + 1 over all
    entries; cells no entry names hold 0 / 0.0; for a repeated (slot, id) the
    entry listed last wins. An empty list gives None; a slot or id out of
    range raises ValueError. Returns (a, b, s, n_adapters, n_experts) with
    flat lists."""
    if len(entries) == 0:
        return None
    for sl, e, _, _, _ in entries:
        if not (0 <= int(sl) <= MAX_ADAPTER_SLOT) or not (0 <= int(e) <= MAX_EXPERT_ID):
            raise ValueError(f"slot {sl} / expert id {e} out of range")
    n_ad = max(int(sl) for sl, *_ in entries) + 1
    n_ex = max(int(e) for _, e, *_ in entries) + 1
    a = [0] * (n_ad * n_ex)
    b = [0] * (n_ad * n_ex)
    s = [0.0] * (n_ad * n_ex)
    for sl, e, aa, bb, sc in entries:
        c = int(sl) * n_ex + int(e)
        a[c], b[c], s[c] = int(aa), int(bb), sc
    return a, b, s, n_ad, n_ex


def fold_gather_multi(x: np.ndarray, a_table, b_table, scale_table, n_adapters: int,
                      n_experts: int, mats, base: np.ndarray, indices, row_adapter,
                      top_k: int) -> np.ndarray:
    """Multi-adapter gather fold, one row at a time: row r with token
    t = r // top_k folds with cell (row_adapter[t], indices[r])."""
    out = np.array(base, dtype=np.float64, copy=True)
    for row in range(len(indices)):
        t = row // top_k
        slot = int(row_adapter[t])
        if slot < 0 or slot >= n_adapters:
            continue
        e = int(indices[row])
        if e < 0 or e >= n_experts:
            continue
        c = slot * n_experts + e
        if a_table[c] == 0 or b_table[c] == 0:
            continue
        a = mats[a_table[c]]
        b = mats[b_table[c]]
        out[row] = base[row] + float(scale_table[c]) * (b @ (a @ x[t]))
    return out
