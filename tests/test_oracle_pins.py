"""Pins for the oracle: checks against facts the pages and the mathematics fix,
not against the oracle itself.

* golden fixtures (tests/golden), each citing the page item it restates;
* hand-worked folds with the arithmetic written out in the fixture;
* closed forms (one-hot rank-1 fold), special cases that reduce to a textbook
  formula (the one-entry router route is dense LoRA, checked through the merged
  weight ``scale * B @ A``), and invariants (B = 0, linearity in the scale,
  grouped == gather on permuted rows, window splits, skip rules);
* mutation checks: plausible mistakes planted in copies of the oracle must each
  fail at least one of these pins.
"""
from __future__ import annotations

import json
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests.common import OracleView, golden_json, golden_lines
import workloads
from workloads import make_gather_case, make_grouped_case

# ---------------------------------------------------------------------------
# host integer functions
# ---------------------------------------------------------------------------


def test_route_truth_table():
    for line in golden_lines("route_truth_table.txt"):
        slot, active, has, want = line.split()
        assert oracle.resolve_moe_lora_route(int(slot), int(active), bool(int(has))) == want, line


def test_ensure_decode_route_servable():
    oracle.ensure_decode_route_servable(oracle.FOLD)
    oracle.ensure_decode_route_servable(oracle.SKIP)
    with pytest.raises(oracle.RefuseError, match="batch of its own"):
        oracle.ensure_decode_route_servable(oracle.REFUSE)


def test_row_adapter_host_golden():
    for line in golden_lines("row_adapter_host.txt"):
        c = json.loads(line)
        assert oracle.build_moe_row_adapter_host(c["cu"], c["slots"]) == c["expect"], line


def test_row_adapter_decode_golden():
    for line in golden_lines("row_adapter_decode.txt"):
        c = json.loads(line)
        got = oracle.build_moe_row_adapter_decode(c["slots"], c["padded_n"], c["active"], c["has"])
        assert got == c["expect"], line


def test_pack_golden():
    for line in golden_lines("pack_expert_tables.txt"):
        c = json.loads(line)
        got = oracle.pack_expert_tables([tuple(e) for e in c["entries"]])
        if c["expect"] is None:
            assert got is None
            continue
        a, b, s, n = got
        assert (a, b, s, n) == (c["expect"]["a"], c["expect"]["b"], c["expect"]["s"],
                                c["expect"]["n"]), line


def test_pack_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.pack_expert_tables([(-1, 1, 2, 1.0)])
    with pytest.raises(ValueError):
        oracle.pack_expert_tables([(oracle.MAX_EXPERT_ID + 1, 1, 2, 1.0)])


@settings(max_examples=200, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 40), st.integers(0, 2**64 - 1),
                          st.integers(0, 2**64 - 1), st.floats(-4, 4, width=32)),
                min_size=1, max_size=30))
def test_pack_properties(entries):
    a, b, s, n = oracle.pack_expert_tables(entries)
    assert n == max(e for e, *_ in entries) + 1
    assert len(a) == len(b) == len(s) == n
    last = {}
    for e, aa, bb, sc in entries:
        last[e] = (aa, bb, sc)
    for i in range(n):
        assert (a[i], b[i], s[i]) == last.get(i, (0, 0, 0.0))


def test_windows_and_wc_golden():
    for line in golden_lines("windows.txt"):
        c = json.loads(line)
        if "wc" in c:
            off, end, mt = c["wc"]
            assert oracle.grouped_down_wc(off, end, mt) == c["expect"], line
        elif c["expect"] == "error":
            with pytest.raises(ValueError):
                oracle.grouped_down_windows(c["total"], c["cap"])
        else:
            got = oracle.grouped_down_windows(c["total"], c["cap"])
            assert [list(w) for w in got] == c["expect"], line


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 5000), st.integers(1, 700))
def test_windows_cover_exactly(total, cap):
    w = oracle.grouped_down_windows(total, cap)
    covered = []
    for s, e in w:
        assert 0 < e - s <= cap
        covered.extend(range(s, e))
    assert covered == list(range(total))
    # greedy: every window but the last is full
    assert all(e - s == cap for s, e in w[:-1])


def test_row_token():
    assert oracle.gather_row_token(0, 8) == 0
    assert oracle.gather_row_token(7, 8) == 0
    assert oracle.gather_row_token(8, 8) == 1
    assert oracle.gather_row_token(639, 8) == 79
    assert oracle.gather_row_token(5, 1) == 5


# ---------------------------------------------------------------------------
# fold pins, written against a pluggable implementation so the mutation test
# can run them on mistaken copies of the oracle
# ---------------------------------------------------------------------------


def _hand():
    g = golden_json("fold_hand.json")
    x = np.array(g["x"], dtype=np.float64)
    mats = {}
    for name, m in g["A"].items():
        mats[100 + int(name)] = np.array(m, dtype=np.float64)
    for name, m in g["B"].items():
        mats[200 + int(name)] = np.array(m, dtype=np.float64)
    entries = []
    for e, a, b, s in g["entries"]:
        entries.append((e, 0 if a is None else 100 + int(a[1:]),
                        0 if b is None else 200 + int(b[1:]), s))
    a_t, b_t, s_t, _ = oracle.pack_expert_tables(entries)
    return g, x, mats, a_t, b_t, s_t, np.array(g["base"], dtype=np.float64)


def pin_gather_hand(gather):
    g, x, mats, a_t, b_t, s_t, base = _hand()
    for c in g["gather"]:
        got = gather(x, a_t, b_t, s_t, mats, base, c["indices"], c["row_adapter"], g["top_k"])
        if not np.array_equal(got, np.array(c["expect"], dtype=np.float64)):
            return False
    return True


def pin_grouped_hand(grouped):
    g, x, mats, a_t, b_t, s_t, base = _hand()
    for c in g["grouped"]:
        lo, hi = c["window"]
        got = grouped(x, a_t, b_t, s_t, mats, base, c["expert_offsets"], c["sorted_ids"],
                      c["row_adapter"], g["top_k"], lo, hi)
        if not np.array_equal(got, np.array(c["expect"], dtype=np.float64)):
            return False
    return True


def pin_gather_x_by_row_hand(gather_rows):
    """Hand-worked folds in the slot-major x mode (fold_hand.json,
    gather_x_by_row): each flat row reads x at its own index."""
    g, _, mats, a_t, b_t, s_t, base = _hand()
    for c in g["gather_x_by_row"]:
        x = np.array(c["x"], dtype=np.float64)
        got = gather_rows(x, a_t, b_t, s_t, mats, base, c["indices"], c["row_adapter"],
                          g["top_k"])
        if not np.array_equal(got, np.array(c["expect"], dtype=np.float64)):
            return False
    return True


def test_gather_x_by_row_pin():
    for fold in (oracle.fold_gather, oracle.fold_gather_scalar):
        assert pin_gather_x_by_row_hand(
            lambda *a: fold(*a, x_rows="row"))


def test_gather_x_by_row_token_mutant_is_caught():
    """Reading x at the token (the default mode) in the slot-major mode fails
    the hand-worked pin."""
    assert not pin_gather_x_by_row_hand(lambda *a: oracle.fold_gather(*a, x_rows="token"))


def test_gather_x_by_row_equals_token_mode_on_repeated_rows():
    """Slot-major x that repeats each token's row top_k times folds exactly as
    token-major x."""
    v = _small_gather(seed=14)
    c = v.case
    x_slot = np.repeat(v.x, c.top_k, axis=0)[: c.n_rows]
    base = np.random.default_rng(8).standard_normal((c.n_rows, 4))
    a = oracle.fold_gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base, c.indices,
                           v.row_adapter, c.top_k)
    b = oracle.fold_gather(x_slot, v.a_table, v.b_table, v.scale_table, v.mats, base, c.indices,
                           v.row_adapter, c.top_k, x_rows="row")
    assert np.array_equal(a, b)


def _small_gather(seed=11, **kw):
    args = dict(n_seq=6, padded_n=8, top_k=3, n_route=7, k_in=5, n_out=4, max_rank=2,
                dtype="f32", n_adapted=5, skip_seqs=1)
    args.update(kw)
    return OracleView(make_gather_case(seed, **args))


def pin_gather_b_zero(gather):
    v = _small_gather()
    mats = {k: (np.zeros_like(m) if m.shape == (4, 2) else m) for k, m in v.mats.items()}
    base = np.random.default_rng(0).standard_normal((v.case.n_rows, 4))
    got = gather(v.x, v.a_table, v.b_table, v.scale_table, mats, base, v.case.indices,
                 v.row_adapter, v.case.top_k)
    return bool(np.all(got == base))


def pin_gather_rank1_onehot(gather):
    """One-hot token rows and rank 1: the delta of a row with token t, expert e
    and x[t] = unit vector i is scale_e * A_e[0, i] * B_e[:, 0]."""
    rng = np.random.default_rng(5)
    top_k, n_tok, k_in, n_out, n_exp = 2, 4, 6, 3, 3
    x = np.zeros((n_tok, k_in))
    hot = [4, 0, 2, 5]
    for t, i in enumerate(hot):
        x[t, i] = 1.0
    mats, entries = {}, []
    for e in range(n_exp):
        mats[10 + e] = rng.standard_normal((1, k_in))
        mats[20 + e] = rng.standard_normal((n_out, 1))
        entries.append((e, 10 + e, 20 + e, float(e + 1) * 0.75))
    a_t, b_t, s_t, _ = oracle.pack_expert_tables(entries)
    idx = [0, 2, 1, 1, 2, 0, 0, 1]
    base = np.zeros((len(idx), n_out))
    got = gather(x, a_t, b_t, s_t, mats, base, idx, [1] * n_tok, top_k)
    for row, e in enumerate(idx):
        t = row // top_k
        want = s_t[e] * mats[10 + e][0, hot[t]] * mats[20 + e][:, 0]
        if not np.allclose(got[row], want, rtol=1e-14, atol=0.0):
            return False
    return True


def pin_gather_scale_linear(gather):
    """Doubling every scale doubles every delta exactly (base 0)."""
    v = _small_gather(seed=12)
    base = np.zeros((v.case.n_rows, 4))
    d1 = gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base, v.case.indices,
                v.row_adapter, v.case.top_k)
    s2 = [2.0 * s for s in v.scale_table]
    d2 = gather(v.x, v.a_table, v.b_table, s2, v.mats, base, v.case.indices,
                v.row_adapter, v.case.top_k)
    return bool(np.array_equal(d2, 2.0 * d1)) and bool(np.any(d1 != 0))


def pin_router_dense_lora(gather):
    """A one-entry route with top_k = 1 and every row on expert 0 is dense LoRA;
    checked through the merged weight delta_W = scale * B @ A."""
    rng = np.random.default_rng(9)
    t, k_in, n_out, r = 9, 7, 5, 3
    x = rng.standard_normal((t, k_in))
    a = rng.standard_normal((r, k_in))
    b = rng.standard_normal((n_out, r))
    s = 1.25
    base = rng.standard_normal((t, n_out))
    a_t, b_t, s_t, _ = oracle.pack_expert_tables([(0, 1, 2, s)])
    got = gather(x, a_t, b_t, s_t, {1: a, 2: b}, base, [0] * t, [0] * t, 1)
    w_delta = s * (b @ a)               # [n_out, k_in]
    want = base + x @ w_delta.T
    return bool(np.allclose(got, want, rtol=1e-12, atol=1e-12))


def pin_gather_integer_bruteforce(gather):
    """Small integer inputs: exact rational brute force (every product and sum
    written out) equals the fp64 result bit for bit."""
    rng = np.random.default_rng(21)
    top_k, n_tok, k_in, n_out, r, n_exp = 2, 3, 4, 3, 2, 3
    x = rng.integers(-2, 3, (n_tok, k_in)).astype(np.float64)
    mats, entries = {}, []
    for e in range(n_exp):
        mats[10 + e] = rng.integers(-2, 3, (r, k_in)).astype(np.float64)
        mats[20 + e] = rng.integers(-2, 3, (n_out, r)).astype(np.float64)
        entries.append((e, 10 + e, 20 + e, [0.5, 1.0, 2.0][e]))
    a_t, b_t, s_t, _ = oracle.pack_expert_tables(entries)
    idx = [2, 0, 1, 2, 0, 1]
    ra = [1, -1, 1]
    base = rng.integers(-3, 4, (len(idx), n_out)).astype(np.float64)
    got = gather(x, a_t, b_t, s_t, mats, base, idx, ra, top_k)
    for row, e in enumerate(idx):
        t = row // top_k
        for n in range(n_out):
            acc = Fraction(int(base[row, n]))
            if ra[t] >= 0:
                for j in range(r):
                    h = sum(Fraction(int(mats[10 + e][j, k])) * Fraction(int(x[t, k]))
                            for k in range(k_in))
                    acc += Fraction(s_t[e]) * Fraction(int(mats[20 + e][n, j])) * h
            if Fraction(got[row, n]) != acc:
                return False
    return True


def pin_gather_skips(gather):
    """Rows with a negative map entry, a null cell (a only, b only, both), an id
    at/after the table length or a negative id are returned bit for bit; a
    live row on the same tables changes."""
    rng = np.random.default_rng(3)
    k_in, n_out, r, top_k = 4, 3, 2, 1
    x = rng.standard_normal((7, k_in))
    # address 0 holds junk: an implementation that reads a null cell uses it
    mats = {0: rng.standard_normal((n_out, r)), 1: rng.standard_normal((r, k_in)),
            2: rng.standard_normal((n_out, r))}
    entries = [(0, 1, 2, 1.0), (1, 0, 2, 1.0), (2, 1, 0, 1.0), (3, 0, 0, 0.0), (4, 1, 2, 1.0)]
    a_t, b_t, s_t, _ = oracle.pack_expert_tables(entries)
    idx = [1, 2, 3, 5, -1, 0, 4]
    ra = [0, 0, 0, 0, 0, -1, 0]
    base = rng.standard_normal((7, n_out))
    got = gather(x, a_t, b_t, s_t, mats, base, idx, ra, top_k)
    untouched = got[:6].view(np.uint64) == base[:6].view(np.uint64)
    return bool(np.all(untouched)) and bool(np.all(got[6] != base[6]))


def pin_gather_scalar_equals_vectorized(gather):
    v = _small_gather(seed=13, wild_index_frac=0.2)
    base = np.random.default_rng(1).standard_normal((v.case.n_rows, 4))
    got = gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base, v.case.indices,
                 v.row_adapter, v.case.top_k)
    ref = oracle.fold_gather_scalar(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base,
                                    v.case.indices, v.row_adapter, v.case.top_k)
    return bool(np.allclose(got, ref, rtol=1e-12, atol=1e-12))


GATHER_PINS = [pin_gather_hand, pin_gather_b_zero, pin_gather_rank1_onehot,
               pin_gather_scale_linear, pin_router_dense_lora, pin_gather_integer_bruteforce,
               pin_gather_skips, pin_gather_scalar_equals_vectorized]


def _small_grouped(seed=31, **kw):
    args = dict(stream_lens=[5, 0, 7, 4], top_k=3, n_route=6, k_in=5, n_out=4, max_rank=2,
                dtype="f32", n_unadapted=2, dup_frac=0.3, cap=7,
                stream_slot_values=[1, 1, -1, 1])
    args.update(kw)
    return OracleView(make_grouped_case(seed, **args))


def pin_grouped_equals_gather_permuted(grouped):
    """Grouped row r equals gather row sorted_ids[r] on the same inputs."""
    v = _small_grouped()
    c = v.case
    base_flat = np.random.default_rng(2).standard_normal((c.n_rows, 4))
    base_sorted = base_flat[c.sorted_ids]
    out_g = grouped(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base_sorted,
                    c.expert_offsets, c.sorted_ids, v.row_adapter, c.top_k, 0, c.n_rows)
    out_flat = oracle.fold_gather(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base_flat,
                                  c.notes["indices_flat"], v.row_adapter, c.top_k)
    return bool(np.allclose(out_g, out_flat[c.sorted_ids], rtol=1e-12, atol=1e-12))


def pin_grouped_windows(grouped):
    """Folding window after window equals folding one window over all rows, and
    rows outside a window stay as given."""
    v = _small_grouped(seed=32)
    c = v.case
    base = np.random.default_rng(4).standard_normal((c.n_rows, 4))
    whole = grouped(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base, c.expert_offsets,
                    c.sorted_ids, v.row_adapter, c.top_k, 0, c.n_rows)
    out = base.copy()
    for s, e in oracle.grouped_down_windows(c.n_rows, 5):
        nxt = grouped(v.x, v.a_table, v.b_table, v.scale_table, v.mats, out, c.expert_offsets,
                      c.sorted_ids, v.row_adapter, c.top_k, s, e)
        outside = np.ones(c.n_rows, dtype=bool)
        outside[s:e] = False
        if not np.array_equal(nxt[outside], out[outside]):
            return False
        out = nxt
    return bool(np.allclose(out, whole, rtol=1e-12, atol=1e-12))


def pin_grouped_spans(grouped):
    """Rows before the first span start or after the last span end fold nothing;
    rows of an empty span's neighbours use the neighbour's expert."""
    g, x, mats, a_t, b_t, s_t, base = _hand()
    got = grouped(x, a_t, b_t, s_t, mats, base, [1, 1, 3, 3], [1, 0, 3, 2], [1, 1], 2, 0, 4)
    want = np.array(g["grouped"][3]["expect"], dtype=np.float64)
    return bool(np.array_equal(got, want))


GROUPED_PINS = [pin_grouped_hand, pin_grouped_equals_gather_permuted, pin_grouped_windows,
                pin_grouped_spans]


@pytest.mark.parametrize("pin", GATHER_PINS, ids=lambda f: f.__name__)
def test_gather_pins(pin):
    assert pin(oracle.fold_gather)
    assert pin(oracle.fold_gather_scalar)


@pytest.mark.parametrize("pin", GROUPED_PINS, ids=lambda f: f.__name__)
def test_grouped_pins(pin):
    assert pin(oracle.fold_grouped)
    assert pin(oracle.fold_grouped_scalar)


def pin_grouped_windows_hand(windows_fold):
    """Hand-worked window lists (tests/golden/fold_hand.json, grouped_windows):
    each window folds on the result of the ones before it."""
    g, x, mats, a_t, b_t, s_t, base = _hand()
    for c in g["grouped_windows"]:
        wins = [tuple(w) for w in c["windows"]]
        got = windows_fold(x, a_t, b_t, s_t, mats, base, c["expert_offsets"], c["sorted_ids"],
                           c["row_adapter"], g["top_k"], wins)
        if not np.array_equal(got, np.array(c["expect"], dtype=np.float64)):
            return False
    return True


def _windows_mutant(kind):
    def f(x, a_table, b_table, scale_table, mats, base, expert_offsets, sorted_ids,
          row_adapter, top_k, windows):
        out = np.array(base, dtype=np.float64, copy=True)
        wins = list(windows)
        if kind == "first_window_only":
            wins = wins[:1]
        for (s, e) in wins:
            src = base if kind == "from_original_base" else out
            out = oracle.fold_grouped(x, a_table, b_table, scale_table, mats, src,
                                      expert_offsets, sorted_ids, row_adapter, top_k, s, e)
        return out
    return f


def test_grouped_windows_pin():
    assert pin_grouped_windows_hand(oracle.fold_grouped_windows)


@pytest.mark.parametrize("kind", ["from_original_base", "first_window_only"])
def test_windows_mutant_is_caught(kind):
    assert not pin_grouped_windows_hand(_windows_mutant(kind))


def test_grouped_scalar_equals_vectorized():
    v = _small_grouped(seed=33)
    c = v.case
    base = np.random.default_rng(6).standard_normal((c.n_rows, 4))
    for s, e in [(0, c.n_rows), (3, 11), (c.n_rows, c.n_rows)]:
        a = oracle.fold_grouped(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base,
                                c.expert_offsets, c.sorted_ids, v.row_adapter, c.top_k, s, e)
        b = oracle.fold_grouped_scalar(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base,
                                       c.expert_offsets, c.sorted_ids, v.row_adapter, c.top_k,
                                       s, e)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_unnamed_rows_fold_nothing():
    """Adding rows that name no token (lead and tail rows outside every span,
    ids of -1 or past the last token inside spans) changes nothing else: every
    row whose id is kept folds as in the original case, every other row is
    returned as given, in the vectorized and the scalar oracle."""
    import workloads
    c = make_grouped_case(35, stream_lens=[9, 6], top_k=3, n_route=5, k_in=6, n_out=4,
                          max_rank=2, dtype="f32", n_unadapted=1, cap=8)
    u = workloads.with_unnamed_rows(c, 35, lead=4, tail=3, bad_frac=0.3)
    vc, vu = OracleView(c), OracleView(u)
    ref_c = vc.fold(windows=[(0, c.n_rows)])
    n_flat = c.n_tokens * c.top_k
    kept = (u.sorted_ids[4:4 + c.n_rows] >= 0) & (u.sorted_ids[4:4 + c.n_rows] < n_flat)
    assert kept.sum() < c.n_rows
    base_u = to_f64_case(u)
    for fold in (oracle.fold_grouped, oracle.fold_grouped_scalar):
        got = fold(vu.x, vu.a_table, vu.b_table, vu.scale_table, vu.mats, base_u,
                   u.expert_offsets, u.sorted_ids, vu.row_adapter, u.top_k, 0, u.n_rows)
        mid = got[4:4 + c.n_rows]
        # fp64, up to the order BLAS adds the products in
        assert np.allclose(mid[kept], ref_c[kept], rtol=1e-13, atol=1e-13)
        assert np.array_equal(mid[~kept], base_u[4:4 + c.n_rows][~kept])
        assert np.array_equal(got[:4], base_u[:4]) and np.array_equal(got[-3:], base_u[-3:])
        live = vu.live_rows()
        assert np.array_equal(live[4:4 + c.n_rows], kept & vc.live_rows())
        assert not live[:4].any() and not live[-3:].any()


def to_f64_case(case):
    from tests.common import to_f64
    return to_f64(case.base, case.dtype)


def test_decoy_entries_lose():
    """With duplicate ids packed decoy-first, the fold equals the fold of the
    real entries alone (the last duplicate wins)."""
    v = _small_grouped(seed=34, dup_frac=0.5)
    c = v.case
    seen, real = set(), []
    for ent in reversed(v.entries):
        if ent[0] not in seen:
            seen.add(ent[0])
            real.append(ent)
    a2, b2, s2, _ = oracle.pack_expert_tables(list(reversed(real)))
    assert len(real) < len(v.entries)
    base = np.random.default_rng(7).standard_normal((c.n_rows, 4))
    x1 = oracle.fold_grouped(v.x, v.a_table, v.b_table, v.scale_table, v.mats, base,
                             c.expert_offsets, c.sorted_ids, v.row_adapter, c.top_k, 0, c.n_rows)
    x2 = oracle.fold_grouped(v.x, a2, b2, s2, v.mats, base, c.expert_offsets, c.sorted_ids,
                             v.row_adapter, c.top_k, 0, c.n_rows)
    assert np.array_equal(x1, x2)


# ---------------------------------------------------------------------------
# mutation checks: each planted mistake must fail at least one pin
# ---------------------------------------------------------------------------


def _gather_mutant(kind):
    def f(x, a_table, b_table, scale_table, mats, base, indices, row_adapter, top_k):
        out = np.array(base, dtype=np.float64, copy=True)
        n = len(a_table)
        for row in range(len(indices)):
            t = row if kind == "token_is_row" else row // top_k
            t = min(t, x.shape[0] - 1)
            gate = row_adapter[min(row, len(row_adapter) - 1)] if kind == "map_by_row" \
                else row_adapter[t]
            if kind != "no_map_check" and gate < 0:
                continue
            e = int(indices[row])
            if kind == "no_b_cell_check":
                ok = 0 <= e < n and a_table[e] != 0
            elif kind == "signed_only_upper":
                ok = e < n and a_table[e] != 0 and b_table[e] != 0
            else:
                ok = 0 <= e < n and a_table[e] != 0 and b_table[e] != 0
            if not ok:
                continue
            a = mats[a_table[e]]
            b = mats[b_table[e]]
            if kind == "a_transposed_use":
                h = (x[t] @ a.T[:, :]) if a.shape[1] == x.shape[1] else None
                h = a[:, ::-1] @ x[t]
            else:
                h = a @ x[t]
            s = 1.0 if kind == "no_scale" else float(scale_table[e])
            delta = s * (b @ h)
            if kind == "minus":
                delta = -delta
            if kind == "square_h":
                delta = s * (b @ (h * h))
            out[row] = base[row] + delta
        return out
    return f


GATHER_MUTANTS = ["token_is_row", "map_by_row", "no_map_check", "no_b_cell_check",
                  "signed_only_upper", "a_transposed_use", "no_scale", "minus", "square_h"]


@pytest.mark.parametrize("kind", GATHER_MUTANTS)
def test_gather_mutant_is_caught(kind):
    mut = _gather_mutant(kind)
    results = []
    for pin in GATHER_PINS:
        try:
            results.append(pin(mut))
        except Exception:
            results.append(False)
    assert not all(results), f"mutant {kind} passed every pin"


def _grouped_mutant(kind):
    def f(x, a_table, b_table, scale_table, mats, base, expert_offsets, sorted_ids,
          row_adapter, top_k, row_offset, row_end):
        out = np.array(base, dtype=np.float64, copy=True)
        off = [int(v) for v in expert_offsets]
        hi = row_end + 1 if kind == "window_inclusive" else row_end
        for r in range(row_offset, min(hi, len(base))):
            owner = -1
            for e in range(len(off) - 1):
                inside = off[e] <= r <= off[e + 1] if kind == "closed_span" \
                    else off[e] <= r < off[e + 1]
                if inside:
                    owner = e
                    break
            if owner < 0:
                if kind == "orphan_to_zero":
                    owner = 0
                else:
                    continue
            rid = int(sorted_ids[r])
            if kind == "token_is_sorted_row":
                t = r // top_k
            elif kind == "token_is_id":
                t = min(rid, x.shape[0] - 1)
            elif kind == "no_id_check":
                t = rid // top_k  # a negative id wraps to the last token
            elif kind == "clip_token":
                t = min(max(rid // top_k, 0), x.shape[0] - 1)
            else:
                if rid < 0 or rid // top_k >= x.shape[0]:
                    continue
                t = rid // top_k
            if row_adapter[t] < 0:
                continue
            e = owner
            if not (0 <= e < len(a_table) and a_table[e] != 0 and b_table[e] != 0):
                continue
            a, b = mats[a_table[e]], mats[b_table[e]]
            out[r] = base[r] + float(scale_table[e]) * (b @ (a @ x[t]))
        return out
    return f


GROUPED_MUTANTS = ["window_inclusive", "closed_span", "orphan_to_zero", "token_is_sorted_row",
                   "token_is_id", "no_id_check", "clip_token"]


@pytest.mark.parametrize("kind", GROUPED_MUTANTS)
def test_grouped_mutant_is_caught(kind):
    mut = _grouped_mutant(kind)
    results = []
    for pin in GROUPED_PINS:
        try:
            results.append(pin(mut))
        except Exception:
            results.append(False)
    assert not all(results), f"mutant {kind} passed every pin"


def test_pack_mutants_are_caught():
    """First-duplicate-wins and table length = max id both fail the golden file."""
    def first_wins(entries):
        if not entries:
            return None
        n = max(e for e, *_ in entries) + 1
        a, b, s = [0] * n, [0] * n, [0.0] * n
        for e, aa, bb, sc in reversed(list(entries)):
            a[e], b[e], s[e] = aa, bb, sc
        return a, b, s, n

    def short_table(entries):
        if not entries:
            return None
        n = max(e for e, *_ in entries)
        a, b, s = [0] * (n + 1), [0] * (n + 1), [0.0] * (n + 1)
        for e, aa, bb, sc in entries:
            a[e], b[e], s[e] = aa, bb, sc
        return a, b, s, n

    for mut in (first_wins, short_table):
        ok = True
        for line in golden_lines("pack_expert_tables.txt"):
            c = json.loads(line)
            got = mut([tuple(e) for e in c["entries"]])
            want = None if c["expect"] is None else (
                c["expect"]["a"], c["expect"]["b"], c["expect"]["s"], c["expect"]["n"])
            ok &= got == want
        assert not ok


# ---------------------------------------------------------------------------
# bf16 decoding, from the format's definition
# ---------------------------------------------------------------------------


def _bf16_by_definition(bits: int) -> float:
    """bf16 is 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits:
    normal numbers are (-1)^s 2^(E-127) (1 + f/128), subnormals (E = 0)
    (-1)^s 2^-126 (f/128), E = 255 with f = 0 is infinity."""
    s, e, f = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    sign = -1.0 if s else 1.0
    if e == 255:
        return sign * math.inf
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_known_values():
    got = oracle.bf16_to_f64(np.array([0x3F80, 0xC040, 0x0001, 0x7F7F, 0x0080, 0x3F81,
                                       0x8000, 0x7F80, 0xFF80], dtype=np.uint16))
    assert got[0] == 1.0
    assert got[1] == -3.0
    assert got[2] == 2.0 ** -133            # smallest subnormal
    assert got[3] == (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite
    assert got[4] == 2.0 ** -126            # smallest normal
    assert got[5] == 1.0 + 2.0 ** -7        # one ulp above 1
    assert got[6] == 0.0 and np.signbit(got[6])
    assert got[7] == math.inf and got[8] == -math.inf


def test_bf16_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    got = oracle.bf16_to_f64(bits[finite].astype(np.uint16))
    want = np.array([_bf16_by_definition(int(b)) for b in bits[finite]])
    assert np.array_equal(got.view(np.uint64), want.view(np.uint64))


# ---------------------------------------------------------------------------
# the tolerance reading
# ---------------------------------------------------------------------------


def test_max_abs_reading_on_gateup():
    """On the gate/up gather workload the exact result reaches |v| >= 8, where
    half a bf16 ulp (2**-5) already exceeds 3e-2: the correctly rounded result
    (the best any bf16 output can do) misses a literal 3e-2 bound and meets
    the reading max(3e-2, ulp/2 at |ref| + eps, plus eps). The reading stays
    tighter than one full ulp: a result one ulp off where |ref| >= 8 fails it,
    and the evaluation margin eps is a small fraction of an ulp there."""
    import workloads
    from tests.common import (MAX_ABS_TOL, REL_L2_TOL, max_abs, max_abs_excess, rel_l2,
                              to_f64, ulp, view_margin)
    c = workloads.gateup_gather()
    view = OracleView(c)
    ref = view.fold()
    eps = view_margin(view, ref)
    best = to_f64(workloads.bf16_from_f32(ref.astype(np.float32)), "bf16")
    assert np.abs(ref).max() >= 8.0
    assert max_abs(best, ref) > MAX_ABS_TOL
    assert max_abs_excess(best, ref, "bf16", eps) <= 1.0
    assert rel_l2(best, ref) <= REL_L2_TOL
    big = np.abs(ref) >= 8.0
    assert float(np.max(eps[big] / ulp(ref[big], "bf16"))) < 0.25
    # the far neighbour of the largest element: one full ulp from its exact value
    i = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    off = best.copy()
    off[i] = ref[i] + np.sign(ref[i]) * ulp(np.array([ref[i]]), "bf16")[0]
    assert max_abs_excess(off, ref, "bf16", eps) > 1.0


def test_eval_margin_covers_fp32_evaluation():
    """A plain fp32 evaluation of the fold (the shrink and expand summed in
    fp32, one term at a time, H not rounded) differs from the exact result by
    far less than the margin eps, element by element, on a case where the
    magnitudes are largest (the gate/up shapes: k_in 2048, rank 64)."""
    from tests.common import to_f64, view_margin
    c = make_gather_case(40, n_seq=4, padded_n=4, top_k=8, n_route=16, k_in=2048, n_out=64,
                         max_rank=64, scale=(0.25, 4.0))
    view = OracleView(c)
    ref = view.fold()
    eps = view_margin(view, ref)
    x32 = view.x.astype(np.float32)
    out = ref.copy()
    for row in range(c.n_rows):
        e = int(c.indices[row])
        t = row // c.top_k
        if view.row_adapter[t] < 0 or not (0 <= e < view.n_experts) or view.a_table[e] == 0:
            continue
        a = view.mats[view.a_table[e]].astype(np.float32)
        b = view.mats[view.b_table[e]].astype(np.float32)
        h = np.zeros(c.max_rank, dtype=np.float32)
        for k in range(c.k_in):            # sequential fp32 sums
            h = h + a[:, k] * x32[t, k]
        h = np.float32(view.scale_table[e]) * h
        d = np.zeros(c.n_out, dtype=np.float32)
        for j in range(c.max_rank):
            d = d + b[:, j] * h[j]
        out[row] = to_f64(c.base[row], c.dtype) + d
    err = np.abs(out - ref)
    assert np.all(err <= eps)
    assert float(np.max(err / np.maximum(eps, 1e-300))) < 0.2


def test_oracle_view_folds_slot_major_cases_by_row():
    """The fp64 view of a slot-major case (the decode layer's down fold)
    reads x at the flat row, in its fold and in its magnitude fold (the
    tolerance's scale), not at the row's token."""
    import oracle
    from oracle.case import OracleView, to_f64
    down = workloads.decode_layer_cases(seed=7, n_seq=6, padded_n=8, top_k=3, n_route=10,
                                        n_adapted=8, skip_seqs=1, hidden=64, inter=48)[3]
    assert down.notes["x_rows"] == "row"
    view = OracleView(down)
    base = to_f64(down.base, down.dtype)
    args = (view.x, view.a_table, view.b_table, view.scale_table, view.mats, base,
            down.indices, view.row_adapter, down.top_k)
    by_row = oracle.fold_gather(*args, x_rows="row")
    by_token = oracle.fold_gather(*args, x_rows="token")
    assert not np.allclose(by_row, by_token)
    np.testing.assert_array_equal(view.fold(), by_row)
    mats = {k: np.abs(m) for k, m in view.mats.items()}
    mag = oracle.fold_gather(np.abs(view.x), view.a_table, view.b_table,
                             [abs(float(s)) for s in view.scale_table], mats, np.zeros_like(base),
                             down.indices, view.row_adapter, down.top_k, x_rows="row")
    np.testing.assert_array_equal(view.magnitude(), mag)
