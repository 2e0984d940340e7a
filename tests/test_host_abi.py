"""The C ABI without a GPU: the library loads, exports every declared symbol,
and its host-side integer functions match the oracle bit for bit (golden
fixtures plus randomized inputs, malformed ones included). Fold argument
checks that fail before any device work are covered here too."""
from __future__ import annotations

import ctypes
import json
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import moe_expert_lora_amd as ml
import oracle
from tests.common import golden_lines

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ROUTE_NAME = {ml.MLORA_ROUTE_FOLD: oracle.FOLD, ml.MLORA_ROUTE_SKIP: oracle.SKIP,
              ml.MLORA_ROUTE_REFUSE: oracle.REFUSE}


@pytest.fixture(scope="module")
def lib():
    return ml.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "mlora.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mlora_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    decl = declared_functions()
    assert set(decl) == set(ml.EXPORTS), (decl, ml.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_m_tile_matches_header():
    src = open(os.path.join(ROOT, "include", "mlora.h")).read()
    m = re.search(r"#define\s+MLORA_MLG_M_TILE\s+(\d+)", src)
    assert ml.mlora_m_tile() == int(m.group(1))


def test_route_truth_table_golden():
    for line in golden_lines("route_truth_table.txt"):
        slot, active, has, want = line.split()
        got = ml.mlora_resolve_moe_lora_route(int(slot), int(active), bool(int(has)))
        assert ROUTE_NAME[got] == want, line


def test_route_exhaustive_small():
    for slot in range(-3, 5):
        for active in range(-2, 4):
            for has in (False, True):
                got = ml.mlora_resolve_moe_lora_route(slot, active, has)
                assert ROUTE_NAME[got] == oracle.resolve_moe_lora_route(slot, active, has)


def test_ensure_decode_route_servable():
    ml.mlora_ensure_decode_route_servable(ml.MLORA_ROUTE_FOLD)
    ml.mlora_ensure_decode_route_servable(ml.MLORA_ROUTE_SKIP)
    with pytest.raises(ml.MloraError) as ei:
        ml.mlora_ensure_decode_route_servable(ml.MLORA_ROUTE_REFUSE)
    assert ei.value.code == ml.MLORA_ERR_REFUSE
    assert "batch of its own" in str(ei.value)
    with pytest.raises(ml.MloraError) as ei:
        ml.mlora_ensure_decode_route_servable(7)
    assert ei.value.code == ml.MLORA_ERR_INVALID


def _pack_both(entries):
    ids = [e for e, *_ in entries]
    a = [x for _, x, _, _ in entries]
    b = [x for _, _, x, _ in entries]
    s = [x for *_, x in entries]
    got = ml.mlora_pack_expert_tables(ids, a, b, s)
    want = oracle.pack_expert_tables(entries)
    return got, want


def _same_pack(got, want):
    if want is None:
        return got is None
    at, bt, st_, n = got
    wa, wb, ws, wn = want
    return (n == wn and at.tolist() == wa and bt.tolist() == wb
            and st_.view(np.uint32).tolist() == np.asarray(ws, np.float32).view(np.uint32).tolist())


def test_pack_golden():
    for line in golden_lines("pack_expert_tables.txt"):
        c = json.loads(line)
        got, want = _pack_both([tuple(e) for e in c["entries"]])
        assert _same_pack(got, want), line


@settings(max_examples=300, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 300), st.integers(0, 2**64 - 1),
                          st.integers(0, 2**64 - 1),
                          st.floats(allow_nan=False, width=32)), max_size=40))
def test_pack_matches_oracle(entries):
    got, want = _pack_both(entries)
    assert _same_pack(got, want)


def test_pack_rejects_bad_ids():
    for bad in (-1, -100, oracle.MAX_EXPERT_ID + 1, 2**31 - 1):
        with pytest.raises(ml.MloraError) as ei:
            ml.mlora_pack_expert_tables([0, bad], [1, 2], [3, 4], [1.0, 1.0])
        assert ei.value.code == ml.MLORA_ERR_INVALID
    got = ml.mlora_pack_expert_tables([oracle.MAX_EXPERT_ID], [5], [6], [0.5])
    assert got[3] == oracle.MAX_EXPERT_ID + 1 and got[0][-1] == 5


def test_pack_capacity_leaves_tables(lib):
    ids = np.array([3, 1], np.int32)
    a = np.array([11, 12], np.uint64)
    b = np.array([21, 22], np.uint64)
    s = np.array([1.0, 2.0], np.float32)
    at = np.full(2, 99, np.uint64)
    bt = np.full(2, 99, np.uint64)
    stt = np.full(2, 9.0, np.float32)
    n = ctypes.c_int32(-5)
    P = lambda arr, t: arr.ctypes.data_as(ctypes.POINTER(t))  # noqa: E731
    rc = lib.mlora_pack_expert_tables(P(ids, ctypes.c_int32), P(a, ctypes.c_uint64),
                                      P(b, ctypes.c_uint64), P(s, ctypes.c_float), 2,
                                      P(at, ctypes.c_uint64), P(bt, ctypes.c_uint64),
                                      P(stt, ctypes.c_float), 2, ctypes.byref(n))
    assert rc == ml.MLORA_ERR_CAPACITY and n.value == 4
    assert at.tolist() == [99, 99] and stt.tolist() == [9.0, 9.0]


def test_row_adapter_host_golden():
    for line in golden_lines("row_adapter_host.txt"):
        c = json.loads(line)
        got = ml.mlora_build_moe_row_adapter_host(c["cu"], c["slots"])
        if c["expect"] is None:
            assert got is None, line
        else:
            assert got is not None and got.tolist() == c["expect"], line


@settings(max_examples=400, deadline=None)
@given(st.lists(st.integers(-3, 40), max_size=8), st.lists(st.integers(-2, 5), max_size=8),
       st.booleans())
def test_row_adapter_host_matches_oracle(cu, slots, make_valid):
    if make_valid and cu:
        cu = [0] + sorted(abs(v) for v in cu)
        slots = (slots + [1] * len(cu))[: len(cu) - 1]
    got = ml.mlora_build_moe_row_adapter_host(cu, slots)
    want = oracle.build_moe_row_adapter_host(cu, slots)
    if want is None:
        assert got is None
    else:
        assert got is not None and got.tolist() == want


def test_row_adapter_host_none_writes_nothing(lib):
    cu = np.array([0, 4, 2], np.int32)
    sl = np.array([1, 1], np.int32)
    out = np.full(8, 77, np.int32)
    total = ctypes.c_int64(-9)
    rc = lib.mlora_build_moe_row_adapter_host(
        cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 3,
        sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2,
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 8, ctypes.byref(total))
    assert rc == ml.MLORA_NONE
    assert out.tolist() == [77] * 8 and total.value == -9


def test_row_adapter_decode_golden():
    for line in golden_lines("row_adapter_decode.txt"):
        c = json.loads(line)
        got = ml.mlora_build_moe_row_adapter_decode(c["slots"], c["padded_n"], c["active"],
                                                    c["has"])
        assert got.tolist() == c["expect"], line


@settings(max_examples=400, deadline=None)
@given(st.lists(st.integers(-3, 6), max_size=12), st.integers(0, 16), st.integers(-2, 6),
       st.booleans())
def test_row_adapter_decode_matches_oracle(slots, padded_n, active, has):
    got = ml.mlora_build_moe_row_adapter_decode(slots, padded_n, active, has)
    assert got.tolist() == oracle.build_moe_row_adapter_decode(slots, padded_n, active, has)


def test_windows_and_wc_golden():
    for line in golden_lines("windows.txt"):
        c = json.loads(line)
        if "wc" in c:
            off, end, mt = c["wc"]
            if mt == ml.mlora_m_tile():
                assert ml.mlora_grouped_down_wc(off, end) == c["expect"], line
        elif c["expect"] == "error":
            with pytest.raises(ml.MloraError) as ei:
                ml.mlora_grouped_down_windows(c["total"], c["cap"])
            assert ei.value.code == ml.MLORA_ERR_INVALID
        else:
            got = ml.mlora_grouped_down_windows(c["total"], c["cap"])
            assert [list(w) for w in got] == c["expect"], line


@settings(max_examples=400, deadline=None)
@given(st.integers(0, 100000), st.integers(1, 20000))
def test_windows_match_oracle(total, cap):
    assert ml.mlora_grouped_down_windows(total, cap) == oracle.grouped_down_windows(total, cap)


@settings(max_examples=400, deadline=None)
@given(st.integers(0, 10**7), st.integers(-100, 10**5))
def test_wc_matches_oracle(off, length):
    m = ml.mlora_m_tile()
    assert ml.mlora_grouped_down_wc(off, off + length) == oracle.grouped_down_wc(off, off + length, m)


def test_windows_negative_cap():
    for cap in (0, -1):
        with pytest.raises(ml.MloraError):
            ml.mlora_grouped_down_windows(10, cap)


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 2**31 - 1), st.integers(1, 64))
def test_row_token_matches_oracle(row, top_k):
    assert ml.mlora_gather_row_token(row, top_k) == oracle.gather_row_token(row, top_k)


def test_row_token_invalid():
    assert ml.mlora_gather_row_token(3, 0) == -1
    assert ml.mlora_gather_row_token(-1, 2) == -1


# ---- fold argument checks that fail before any device work ----------------

def _route(**kw):
    f = dict(a_table=1 << 20, b_table=1 << 21, scale_table=1 << 22, n_experts=4, k_in=64,
             n_out=32, max_rank=8, dtype=ml.MLORA_BF16)
    f.update(kw)
    return ml.ExpertRoute(f["a_table"], f["b_table"], f["scale_table"], f["n_experts"],
                          f["k_in"], f["n_out"], f["max_rank"], f["dtype"])


FAKE = 1 << 24  # never dereferenced: every call below is rejected before launch


@pytest.mark.parametrize("kw", [dict(k_in=60), dict(n_out=0), dict(max_rank=0),
                                dict(max_rank=129), dict(dtype=7), dict(n_experts=-1),
                                dict(a_table=0)])
def test_gather_rejects_bad_route(lib, kw):
    r = _route(**kw)
    rc = lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, 8, 2, None, 0, None)
    assert rc == ml.MLORA_ERR_INVALID
    assert ml.load().mlora_last_error()


def test_gather_rejects_bad_args(lib):
    r = _route()
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, 8, 0, None, 0, None) == -1
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 3, FAKE, FAKE, FAKE, 8, 2, None, 0, None) == -1
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, -1, 2, None, 0, None) == -1
    assert lib.mlora_gather_bgmv(ctypes.byref(r), None, 4, FAKE, FAKE, FAKE, 8, 2, None, 0, None) == -1
    # nothing to fold: accepted without touching the device
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 0, FAKE, FAKE, FAKE, 0, 2, None, 0, None) == 0
    # workspace: NULL with a size, misaligned, too small
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, 8, 2, None, 256,
                                 None) == -1
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, 8, 2, FAKE + 16,
                                 1 << 20, None) == -1
    need = lib.mlora_gather_bgmv_workspace_bytes(8, r.k_in, r.max_rank)
    assert lib.mlora_gather_bgmv(ctypes.byref(r), FAKE, 4, FAKE, FAKE, FAKE, 8, 2, FAKE,
                                 need - 1, None) == ml.MLORA_ERR_CAPACITY
    r0 = _route(n_experts=0)
    assert lib.mlora_gather_bgmv(ctypes.byref(r0), FAKE, 4, FAKE, FAKE, FAKE, 8, 2, None, 0, None) == 0


def test_grouped_rejects_bad_args(lib):
    r = _route()
    call = lambda **k: lib.mlora_grouped_down(  # noqa: E731
        ctypes.byref(k.get("route", r)), FAKE, k.get("n_tok", 4), FAKE, k.get("n_rows", 8),
        FAKE, k.get("n_route", 4), FAKE, FAKE, k.get("top_k", 2), k.get("off", 0),
        k.get("end", 8), k.get("ws", None), k.get("ws_bytes", 0), None)
    assert call(top_k=0) == -1
    assert call(off=5, end=4) == -1
    assert call(end=9) == -1
    assert call(off=-1) == -1
    assert call(n_route=-1) == -1
    assert call(n_tok=-1) == -1
    assert call(route=_route(max_rank=200)) == -1
    assert call(off=3, end=3) == 0          # empty window
    assert call(n_route=0) == 0             # no spans
    # workspace: NULL with a size, misaligned, too small
    assert call(ws_bytes=256) == -1
    assert call(ws=FAKE + 16, ws_bytes=1 << 20) == -1
    need = lib.mlora_grouped_down_workspace_bytes(0, 8, 16)
    assert call(ws=FAKE, ws_bytes=need - 1) == ml.MLORA_ERR_CAPACITY


def test_grouped_all_rejects_bad_args(lib):
    r = _route()
    call = lambda **k: lib.mlora_grouped_down_all(  # noqa: E731
        ctypes.byref(k.get("route", r)), FAKE, 4, FAKE, k.get("n_rows", 8), FAKE,
        k.get("n_route", 4), FAKE, FAKE, k.get("top_k", 2), k.get("cap", 4),
        k.get("ws", FAKE), k.get("ws_bytes", 1 << 20), None)
    assert call(cap=0) == -1 and call(cap=-3) == -1      # the pages' panic on cap == 0
    assert call(top_k=0) == -1
    assert call(n_rows=-1) == -1
    assert call(ws=None, ws_bytes=256) == -1
    assert call(ws=FAKE + 16) == -1
    # one launch of all 8 rows needs one slot of 8 rows (the size query may
    # report more: it also covers one-window launches)
    need = lib.mlora_grouped_down_workspace_bytes(0, 8, 8)
    assert lib.mlora_grouped_down_all_workspace_bytes(8, 4, 8) >= need
    assert call(ws_bytes=need - 1) == ml.MLORA_ERR_CAPACITY
    assert call(ws=None, ws_bytes=0) == ml.MLORA_ERR_CAPACITY   # bf16 needs one
    assert call(n_rows=0) == 0 and call(n_route=0) == 0


def test_grouped_all_workspace_bytes(lib):
    f, g = lib.mlora_grouped_down_all_workspace_bytes, lib.mlora_grouped_down_workspace_bytes
    # a launch covers whole windows, at least 16384 rows of them; two slots
    # when there is more than one launch
    assert f(32768, 8192, 32) == 2 * g(0, 16384, 32)
    assert f(16384, 8192, 16) == g(0, 16384, 16)      # one launch, one slot
    assert f(40000, 8192, 16) == 2 * g(0, 16384, 16)
    assert f(5000, 8192, 32) == g(0, 5000, 32)
    # 547 windows of 30 > 100 rows by default; a lower launch minimum may
    # launch 3 windows at a time (two slots of 90 rows)
    assert f(100, 30, 100) == 2 * g(0, 90, 100)
    assert f(70000, 6000, 16) == 2 * g(0, 18000, 16)  # three windows per launch
    assert f(100000, 20000, 16) == 2 * g(0, 20000, 16)
    # 1.5 windows: one launch of 12288 rows, or two one-window slots when a
    # launch group would pass 4 GiB of base_out; the size covers both
    assert f(12288, 8192, 16) == max(g(0, 12288, 16), 2 * g(0, 8192, 16))
    assert f(0, 10, 16) == 0 and f(10, 0, 16) == 0 and f(10, 10, 0) == 0


def test_grouped_all_window_fallback_needs_the_queried_size(lib):
    """1.5 windows of a base_out so wide (n_out 2^17) that one launch of both
    would pass 4 GiB: the call falls back to one window per launch (two slots
    of 12000 rows), and the queried size is exactly what it asks for."""
    r = _route(n_out=1 << 17, max_rank=16)
    cap, n_rows = 12000, 18000
    g = lib.mlora_grouped_down_workspace_bytes
    need = lib.mlora_grouped_down_all_workspace_bytes(n_rows, cap, 16)
    assert need == 2 * g(0, cap, 16) > g(0, n_rows, 16)
    rc = lib.mlora_grouped_down_all(ctypes.byref(r), FAKE, 4, FAKE, n_rows, FAKE, 4, FAKE,
                                    FAKE, 2, cap, FAKE, need - 1, None)
    assert rc == ml.MLORA_ERR_CAPACITY


def _all_needed(lib, n_rows, cap, max_rank, n_out=64):
    """What mlora_grouped_down_all asks for under the current overrides, read
    from its capacity error (no workspace given: nothing is launched)."""
    import re
    r = _route(n_out=n_out, max_rank=max_rank)
    rc = lib.mlora_grouped_down_all(ctypes.byref(r), FAKE, 4, FAKE, n_rows, FAKE, 4, FAKE,
                                    FAKE, 2, cap, None, 0, None)
    assert rc == ml.MLORA_ERR_CAPACITY
    msg = lib.mlora_last_error().decode()
    return int(re.search(r"(\d+) needed", msg).group(1))


@pytest.mark.parametrize("n_rows,cap,max_rank", [(32768, 8192, 32), (16384, 8192, 16),
                                                 (100, 30, 100), (12288, 8192, 16),
                                                 (70000, 6000, 16), (1203, 40, 48),
                                                 (5000, 8192, 32), (100000, 20000, 16)])
def test_grouped_all_workspace_bytes_covers_every_override(lib, overrides, n_rows, cap,
                                                           max_rank):
    """The size query reads no environment and covers the call under every
    launch minimum (MLORA_ALL_MIN_ROWS, clamped to 1 .. 16384 by the call):
    the largest of those needs is exactly the queried size; the tile and
    unit-order overrides change neither."""
    query = lib.mlora_grouped_down_all_workspace_bytes(n_rows, cap, max_rank)
    needs = []
    n_caps = -(-n_rows // cap)
    for m in [None, 1, 2, 7, 30, 90, 100, 1000, 8191, 8192, 8193, 16383, 16384, 16385,
              100000] + [cap * k for k in range(1, n_caps + 1) if cap * k <= 16384]:
        if m is None:
            overrides.delete("MLORA_ALL_MIN_ROWS")
        else:
            overrides.set("MLORA_ALL_MIN_ROWS", m)
        assert lib.mlora_grouped_down_all_workspace_bytes(n_rows, cap, max_rank) == query
        needs.append(_all_needed(lib, n_rows, cap, max_rank))
    assert max(needs) == query
    # the tile and unit-order overrides change neither the query nor the need
    overrides.delete("MLORA_ALL_MIN_ROWS")
    base_need = _all_needed(lib, n_rows, cap, max_rank)
    for name, values in (("MLORA_EXPAND_XCD", (0, 1)), ("MLORA_EXPAND_MB", (1, 2, 4)),
                         ("MLORA_EXPAND_CW", (2, 4)), ("MLORA_SHRINK_MB", (1, 2, 4))):
        for v in values:
            overrides.set(name, v)
            assert lib.mlora_grouped_down_all_workspace_bytes(n_rows, cap, max_rank) == query
            assert _all_needed(lib, n_rows, cap, max_rank) == base_need
        overrides.delete(name)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """The no-allocation all-windows call refuses a call whose launch slots
    exceed its static scratch before touching the device (no HIP call is
    made, so this runs without a GPU); the limit is the header's."""
    assert ml.NOALLOC_SCRATCH_BYTES == 32 << 20
    r = _route(n_out=8, max_rank=128)
    n_rows = cap = 72000
    need = lib.mlora_grouped_down_all_workspace_bytes(n_rows, cap, 128)
    assert need > ml.NOALLOC_SCRATCH_BYTES
    rc = lib.mlora_grouped_down_all_noalloc(ctypes.byref(r), FAKE, 9000, FAKE, n_rows, FAKE, 4,
                                            FAKE, FAKE, 8, cap, None)
    assert rc == ml.MLORA_ERR_CAPACITY
    msg = lib.mlora_last_error().decode()
    assert "scratch" in msg and str(need) in msg
    # argument errors come first, as for the workspace form
    assert lib.mlora_grouped_down_all_noalloc(ctypes.byref(r), FAKE, 9000, FAKE, n_rows, FAKE,
                                              4, FAKE, FAKE, 8, 0, None) == ml.MLORA_ERR_INVALID


def test_host_loop_rejects_bad_host_spans(lib):
    """The host-loop baseline checks every host span before launching
    anything (no HIP call is made here)."""
    r = _route()
    u64 = ctypes.c_uint64 * 4
    at, bt = u64(16, 32, 48, 64), u64(16, 32, 48, 64)
    for spans in ([0, 3, 2, 4, 6], [0, 2, 4, 6, 99], [-1, 2, 4, 6, 8]):
        off = (ctypes.c_int32 * 5)(*spans)
        rc = lib.mlora_apply_expert_lora_sorted(ctypes.byref(r), FAKE, 4, FAKE, 8, FAKE, off, 4,
                                                at, bt, FAKE, FAKE, 2, None, 0, None)
        assert rc == ml.MLORA_ERR_INVALID, spans
        assert "span" in lib.mlora_last_error().decode()


def _proj(route, **kw):
    f = dict(x=FAKE, x_rows=64, x_ld=64, x_by_row=0, base_out=FAKE, out_ld=32, indices=FAKE,
             row_adapter=FAKE, map_len=64, n_slots=64, top_k=1)
    f.update(kw)
    return ml.Projection(ctypes.pointer(route), f["x"], f["x_rows"], f["x_ld"], f["x_by_row"],
                         f["base_out"], f["out_ld"], f["indices"], f["row_adapter"],
                         f["map_len"], f["n_slots"], f["top_k"])


def test_gather_set_rejects_bad_sets(lib):
    """Every projection is checked before anything is launched (no HIP call
    is made here)."""
    r16, r32, r64 = _route(max_rank=16), _route(max_rank=32), _route(max_rank=64)
    f32 = _route(max_rank=16, dtype=ml.MLORA_F32)

    def call(*projs):
        arr = (ml.Projection * len(projs))(*projs)
        return lib.mlora_gather_bgmv_set(arr, len(projs), None)

    assert lib.mlora_gather_bgmv_set(None, 0, None) == ml.MLORA_ERR_INVALID
    assert call(*[_proj(r16)] * 5) == ml.MLORA_ERR_INVALID            # more than 4
    assert call(_proj(r16), _proj(r64)) == ml.MLORA_ERR_INVALID       # rank blocks differ
    assert "rank blocks" in lib.mlora_last_error().decode()
    assert call(_proj(f32)) == ml.MLORA_ERR_INVALID                   # bf16 only
    assert call(_proj(r16, x_ld=60)) == ml.MLORA_ERR_INVALID          # x_ld < k_in
    assert call(_proj(r16, out_ld=36)) == ml.MLORA_ERR_INVALID        # not a multiple of 8
    assert call(_proj(r16, x_by_row=1, x_rows=63)) == ml.MLORA_ERR_INVALID  # < n_slots
    assert call(_proj(r16, top_k=4, map_len=15)) == ml.MLORA_ERR_INVALID    # < ceil(64 / 4)
    assert call(_proj(r16, base_out=FAKE + 8)) == ml.MLORA_ERR_INVALID      # misaligned
    assert call(_proj(r16), _proj(r16, x=0)) == ml.MLORA_ERR_INVALID        # NULL
    # ranks 17..32 share two rank blocks: a valid mix, rejected here only for
    # its NULL x
    assert call(_proj(r32), _proj(_route(max_rank=24), x=0)) == ml.MLORA_ERR_INVALID
    assert "projection 1" in lib.mlora_last_error().decode()


def test_gather_workspace_bytes(lib):
    f = lib.mlora_gather_bgmv_workspace_bytes
    # KC k ranges (16 k steps each, at most 4) x n_slots x 64 x NB bytes,
    # rounded to 256
    assert f(640, 768, 16) == 2 * 640 * 64       # 24 k steps -> two ranges
    assert f(640, 512, 16) == 1 * 640 * 64       # 16 k steps -> one range
    assert f(2048, 2048, 64) == 4 * 2048 * 64 * 4  # 64 k steps -> 4 ranges
    assert f(8192, 2048, 16) == 4 * 8192 * 64
    assert f(10, 4096, 100) == (4 * 10 * 64 * 8 + 255) // 256 * 256  # capped at 4, NB 7 -> 8
    assert f(3, 64, 8) == 256
    assert f(0, 768, 16) == 0 and f(8, 0, 16) == 0 and f(8, 768, 0) == 0 and f(8, 768, 129) == 0


def test_grouped_workspace_bytes(lib):
    f = lib.mlora_grouped_down_workspace_bytes
    # rows * 64 * NB (NB = ceil(r / 16) rounded up to a power of two), rounded
    # to 256, then 8 bytes per row, rounded
    assert f(0, 8, 16) == 512 + 256
    assert f(0, 8, 100) == 8 * 512 + 256   # 7 rank blocks run as 8
    assert f(0, 8, 48) == 8 * 256 + 256    # 3 rank blocks run as 4
    assert f(10, 20, 17) == 1280 + 256
    assert f(0, 8192, 32) == 8192 * 128 + 8192 * 8
    assert f(0, 1, 128) == 512 + 256
    assert f(5, 5, 16) == 0
    assert f(5, 4, 16) == 0 and f(-1, 4, 16) == 0
    assert f(0, 8, 0) == 0 and f(0, 8, 129) == 0


def test_single_hip_runtime_in_process():
    """The library binds to the HIP runtime PyTorch loaded, not a second copy."""
    import subprocess
    import sys
    code = ("import moe_expert_lora_amd as ml; ml.load(); "
            "maps = open('/proc/self/maps').read(); "
            "print(len({l.split()[-1] for l in maps.splitlines() if 'amdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"


# ---------------------------------------------------------------------------
# multi-adapter host functions against the oracle
# ---------------------------------------------------------------------------

def test_multi_host_golden_through_the_library():
    import json
    import oracle
    from tests.common import golden_lines
    route_name = {ml.MLORA_ROUTE_FOLD: "Fold", ml.MLORA_ROUTE_SKIP: "Skip",
                  ml.MLORA_ROUTE_REFUSE: "Refuse"}
    for line in golden_lines("multi_host.txt"):
        kind, rest = line.split(" ", 1)
        if kind == "route":
            slot, n, want = rest.split()
            assert route_name[ml.mlora_resolve_moe_lora_route_multi(int(slot), int(n))] == want
        elif kind == "decode":
            c = json.loads(rest)
            got = ml.mlora_build_moe_row_adapter_decode_multi(c["slots"], c["padded_n"],
                                                              c["n_adapters"])
            assert got.tolist() == c["expect"], line
        else:
            c = json.loads(rest)
            ent = c["entries"]
            got = ml.mlora_pack_expert_tables_multi([e[0] for e in ent], [e[1] for e in ent],
                                                    [e[2] for e in ent], [e[3] for e in ent],
                                                    [e[4] for e in ent])
            if c["expect"] is None:
                assert got is None
                continue
            at, bt, st, na, ne = got
            e = c["expect"]
            assert (at.tolist(), bt.tolist(), st.tolist(), na, ne) == \
                (e["a"], e["b"], e["s"], e["n_adapters"], e["n_experts"]), line
            assert oracle.pack_expert_tables_multi([tuple(x) for x in ent]) == \
                (e["a"], e["b"], e["s"], e["n_adapters"], e["n_experts"])


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 5), st.integers(0, 30), st.integers(0, 2**64 - 1),
                          st.integers(0, 2**64 - 1), st.floats(-4, 4, width=32)),
                min_size=1, max_size=25),
       st.lists(st.integers(-3, 7), max_size=12), st.integers(0, 14), st.integers(0, 6))
def test_multi_host_fuzz(entries, slots, padded_n, n_adapters):
    import oracle
    got = ml.mlora_pack_expert_tables_multi([e[0] for e in entries], [e[1] for e in entries],
                                            [e[2] for e in entries], [e[3] for e in entries],
                                            [e[4] for e in entries])
    want = oracle.pack_expert_tables_multi(entries)
    at, bt, st_, na, ne = got
    assert (at.tolist(), bt.tolist(), na, ne) == (want[0], want[1], want[3], want[4])
    assert st_.tolist() == [float(np.float32(v)) for v in want[2]]
    m = ml.mlora_build_moe_row_adapter_decode_multi(slots, padded_n, n_adapters)
    assert m.tolist() == oracle.build_moe_row_adapter_decode_multi(slots, padded_n, n_adapters)
    for s_ in slots:
        r = ml.mlora_resolve_moe_lora_route_multi(s_, n_adapters)
        assert {0: "Fold", 1: "Skip", 2: "Refuse"}[r] == \
            oracle.resolve_moe_lora_route_multi(s_, n_adapters)


def test_multi_fold_rejects_bad_calls(lib):
    u64 = FAKE
    r = ml.MultiRoute(u64, u64, u64, 2, 4, 64, 32, 16, ml.MLORA_BF16)

    def call(route, n_tokens=4, n_slots=8, top_k=2, x=FAKE):
        return lib.mlora_gather_bgmv_multi(ctypes.byref(route), x, n_tokens, FAKE, FAKE, FAKE,
                                           n_slots, top_k, None)

    assert call(r, top_k=0) == ml.MLORA_ERR_INVALID
    assert call(r, n_tokens=3) == ml.MLORA_ERR_INVALID          # < ceil(8 / 2)
    assert call(r, x=0) == ml.MLORA_ERR_INVALID
    assert call(ml.MultiRoute(u64, u64, u64, 2, 4, 64, 32, 16, ml.MLORA_F32)) == \
        ml.MLORA_ERR_INVALID                                    # bf16 only
    assert call(ml.MultiRoute(u64, u64, u64, 2, 4, 60, 32, 16, ml.MLORA_BF16)) == \
        ml.MLORA_ERR_INVALID                                    # k_in not a multiple of 8
    assert call(ml.MultiRoute(u64, u64, u64, -1, 4, 64, 32, 16, ml.MLORA_BF16)) == \
        ml.MLORA_ERR_INVALID
    # no cells or no rows: nothing to do, no device access
    assert call(ml.MultiRoute(u64, u64, u64, 0, 4, 64, 32, 16, ml.MLORA_BF16)) == ml.MLORA_OK
    assert call(r, n_slots=0, n_tokens=0) == ml.MLORA_OK
