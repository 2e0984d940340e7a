"""Pins for the multi-adapter oracle (oracle/multi.py): hand-worked folds and
golden host rules, the reduction to the single-adapter fold, the
decomposition into one single-adapter fold per slot, and planted mistakes
that must fail them."""
from __future__ import annotations

import json

import numpy as np
import pytest

import oracle
from tests.common import golden_json, golden_lines
from workloads import make_gather_case
from oracle.case import OracleView


def _hand():
    h = golden_json("fold_hand.json")
    g = golden_json("fold_multi.json")
    x = np.array(h["x"], dtype=np.float64)
    mats = {}
    for name, m in h["A"].items():
        mats[100 + int(name)] = np.array(m, dtype=np.float64)
    for name, m in h["B"].items():
        mats[200 + int(name)] = np.array(m, dtype=np.float64)
    entries = [(sl, e, 0 if a is None else 100 + int(a[1:]), 0 if b is None else 200 + int(b[1:]),
                sc) for sl, e, a, b, sc in g["entries"]]
    base = np.array(h["base"], dtype=np.float64)
    return g, h["top_k"], x, mats, entries, base


def pin_multi_hand(fold):
    g, top_k, x, mats, entries, base = _hand()
    a, b, s, n_ad, n_ex = oracle.pack_expert_tables_multi(entries)
    for c in g["cases"]:
        got = fold(x, a, b, s, n_ad, n_ex, mats, base, c["indices"], c["row_adapter"], top_k)
        if not np.array_equal(got, np.array(c["expect"], dtype=np.float64)):
            return False
    return True


def _two_slot_case(seed=50):
    """A small fp32 case with a second adapter: slot 1's tables reuse the
    weight pool in reverse order, with other scales."""
    v = OracleView(make_gather_case(seed, n_seq=7, padded_n=9, top_k=3, n_route=6, k_in=5,
                                    n_out=4, max_rank=2, dtype="f32", n_adapted=5))
    entries = [(0, e, a, b, s) for (e, a, b, s) in v.entries]
    handles = sorted({a for (_, a, _, _) in v.entries if a})
    for (e, a, b, s) in v.entries:
        if a and b:
            j = handles.index(a)
            a2 = handles[len(handles) - 1 - j]
            entries.append((1, e, a2, a2 + 1, 1.5 * s + 0.25))
    rng = np.random.default_rng(seed)
    ra = rng.choice([-1, 0, 1, 2], size=v.case.padded_n)
    return v, entries, ra


def pin_multi_decomposes_by_slot(fold):
    """The multi fold equals one single-adapter fold per slot, each over the
    rows whose token maps to that slot (the others' map set to -1)."""
    v, entries, ra = _two_slot_case()
    a, b, s, n_ad, n_ex = oracle.pack_expert_tables_multi(entries)
    c = v.case
    base = np.random.default_rng(1).standard_normal((c.n_rows, 4))
    got = fold(v.x, a, b, s, n_ad, n_ex, v.mats, base, c.indices, ra, c.top_k)
    want = base.copy()
    for slot in range(n_ad):
        cells = slice(slot * n_ex, (slot + 1) * n_ex)
        masked = np.where(ra == slot, 0, -1)
        want = oracle.fold_gather(v.x, a[cells], b[cells], s[cells], v.mats, want, c.indices,
                                  masked, c.top_k)
    return bool(np.allclose(got, want, rtol=1e-13, atol=1e-13))


def pin_multi_one_slot_is_single(fold):
    """With one adapter slot, the multi fold is the single-adapter fold on the
    same tables and a map of 0 / -1."""
    v = OracleView(make_gather_case(51, n_seq=8, padded_n=8, top_k=2, n_route=7, k_in=6,
                                    n_out=3, max_rank=2, dtype="f32", n_adapted=6, skip_seqs=2))
    c = v.case
    entries = [(0, e, a, b, s) for (e, a, b, s) in v.entries]
    a, b, s, n_ad, n_ex = oracle.pack_expert_tables_multi(entries)
    ra = np.where(np.asarray(v.row_adapter) >= 0, 0, -1)
    base = np.random.default_rng(2).standard_normal((c.n_rows, 3))
    got = fold(v.x, a, b, s, n_ad, n_ex, v.mats, base, c.indices, ra, c.top_k)
    want = oracle.fold_gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base,
                              c.indices, v.row_adapter, c.top_k)
    return n_ad == 1 and bool(np.allclose(got, want, rtol=1e-13, atol=1e-13))


MULTI_PINS = [pin_multi_hand, pin_multi_decomposes_by_slot, pin_multi_one_slot_is_single]


@pytest.mark.parametrize("pin", MULTI_PINS, ids=lambda f: f.__name__)
def test_multi_pins(pin):
    assert pin(oracle.fold_gather_multi)


def _multi_mutant(kind):
    def f(x, a_table, b_table, scale_table, n_adapters, n_experts, mats, base, indices,
          row_adapter, top_k):
        out = np.array(base, dtype=np.float64, copy=True)
        for row in range(len(indices)):
            t = row // top_k
            slot = int(row_adapter[min(row, len(row_adapter) - 1)] if kind == "slot_by_row"
                       else row_adapter[t])
            if slot < 0:
                continue
            if kind == "slot_ignored":
                slot = 0
            if kind != "no_slot_bound" and slot >= n_adapters:
                continue
            e = int(indices[row])
            if e < 0 or e >= n_experts:
                continue
            c = e * n_adapters + slot if kind == "expert_major" else slot * n_experts + e
            c = min(c, len(a_table) - 1)
            if a_table[c] == 0 or b_table[c] == 0:
                continue
            out[row] = base[row] + float(scale_table[c]) * (
                mats[b_table[c]] @ (mats[a_table[c]] @ x[t]))
        return out
    return f


@pytest.mark.parametrize("kind", ["slot_ignored", "slot_by_row", "no_slot_bound",
                                  "expert_major"])
def test_multi_mutant_is_caught(kind):
    results = []
    for pin in MULTI_PINS:
        try:
            results.append(pin(_multi_mutant(kind)))
        except Exception:
            results.append(False)
    assert not all(results), f"mutant {kind} passed every pin"


def test_multi_host_golden():
    for line in golden_lines("multi_host.txt"):
        kind, rest = line.split(" ", 1)
        if kind == "route":
            slot, n, want = rest.split()
            assert oracle.resolve_moe_lora_route_multi(int(slot), int(n)) == want, line
        elif kind == "decode":
            c = json.loads(rest)
            got = oracle.build_moe_row_adapter_decode_multi(c["slots"], c["padded_n"],
                                                            c["n_adapters"])
            assert got == c["expect"], line
        else:
            c = json.loads(rest)
            got = oracle.pack_expert_tables_multi([tuple(e) for e in c["entries"]])
            if c["expect"] is None:
                assert got is None
            else:
                e = c["expect"]
                assert got == (e["a"], e["b"], e["s"], e["n_adapters"], e["n_experts"]), line


def test_multi_pack_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.pack_expert_tables_multi([(-1, 0, 1, 2, 1.0)])
    with pytest.raises(ValueError):
        oracle.pack_expert_tables_multi([(0, -1, 1, 2, 1.0)])
