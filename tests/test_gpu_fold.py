"""GPU parity of the two folds against the fp64 oracle, through the C ABI.

Bar (per fold call, over the whole base_out tensor): relative L2 <= 2e-3 and
max abs <= 3e-2 against the unrounded fp64 oracle, on a random base (R run)
and on a zero base (Z run, which measures the delta itself). Rows the fold
must not touch are compared bit for bit; integer maps and tables bit for bit.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest

import workloads
from tests.common import REL_L2_TOL, OracleView, parity_figures, to_f64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@functools.lru_cache(maxsize=None)
def staged(name):
    from staging import DeviceCase
    case = workloads.WORKLOADS[name]()
    return case, OracleView(case), DeviceCase(case, DEV)


def put_sentinel(base, rows, dtype):
    """Fill `rows` of base with a signalling-NaN pattern (written through an
    integer view); any arithmetic write would turn it into another pattern."""
    if dtype == "bf16":
        base.view(np.uint16)[rows] = 0x7F81
    else:
        base.view(np.uint32)[rows] = 0x7F800001


def check(view, got, base, label, windows=None):
    ref = view.fold(base=base, windows=windows)
    g = to_f64(got, view.case.dtype)
    rel, mx, ex = parity_figures(view, g, ref, label, windows)
    print(f"{label}: rel_l2={rel:.3e} max_abs={mx:.3e} max_abs/limit={ex:.3f}", flush=True)
    assert rel <= REL_L2_TOL, f"{label}: rel L2 {rel}"
    assert ex <= 1.0, f"{label}: max abs {mx} (ratio to limit {ex})"
    live = view.live_rows()
    if (~live).any():
        assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8)), \
            f"{label}: a row that folds nothing was written"
    return rel, mx


ALL = ["tiny_gather_f32", "decode_down_gather", "prefill_grouped_down", "gateup_gather", "router_gather", "mixed_grouped"]


@pytest.mark.parametrize("name", ALL)
def test_integer_maps_and_tables_bit_exact(name):
    """The map and windows from the library equal the oracle's; the device
    tables hold, cell for cell, the oracle's packing of the same entries with
    the real device addresses of the weights (address and scale bits)."""
    import oracle
    _need_gpu()
    case, view, dev = staged(name)
    assert dev.row_adapter_host.tolist() == view.row_adapter.tolist()
    ids, a_addrs, b_addrs, scales = dev.entries_host
    packed = oracle.pack_expert_tables(
        [(int(e), int(a), int(b), float(s)) for e, a, b, s in zip(ids, a_addrs, b_addrs, scales)])
    oa, ob, os_, on = packed
    at, bt, st, n = dev.tables_host
    assert n == on == view.n_experts
    dev_a = dev.a_table.cpu().numpy().view(np.uint64)[:n]
    dev_b = dev.b_table.cpu().numpy().view(np.uint64)[:n]
    dev_s = dev.scale_table.cpu().numpy()[:n]
    assert dev_a.tolist() == at.tolist() == [int(v) for v in oa]
    assert dev_b.tolist() == bt.tolist() == [int(v) for v in ob]
    want_s = np.asarray(os_, dtype=np.float32).view(np.uint32).tolist()
    assert dev_s.view(np.uint32).tolist() == st.view(np.uint32).tolist() == want_s
    # null cells where the oracle's own view (opaque addresses) has them
    assert [int(v != 0) for v in at] == [int(v != 0) for v in view.a_table]
    assert [int(v != 0) for v in bt] == [int(v != 0) for v in view.b_table]
    if case.path == "grouped":
        assert dev.windows == oracle.grouped_down_windows(case.n_rows, case.cap)


@pytest.mark.parametrize("name", ALL)
def test_parity_random_base(name):
    _need_gpu()
    case, view, dev = staged(name)
    got = dev.run()
    check(view, got, case.base, f"{name} R")


@pytest.mark.parametrize("name", ALL)
def test_parity_zero_base(name):
    _need_gpu()
    case, view, dev = staged(name)
    base = np.zeros_like(case.base)
    got = dev.run(base)
    check(view, got, base, f"{name} Z")


@pytest.mark.parametrize("name", ALL)
def test_untouched_rows_sentinel(name):
    _need_gpu()
    case, view, dev = staged(name)
    live = view.live_rows()
    base = case.base.copy()
    put_sentinel(base, ~live, case.dtype)
    got = dev.run(base)
    assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))
    assert not np.any(np.isnan(to_f64(got[live], case.dtype)))


@pytest.mark.parametrize("name", ["decode_down_gather", "prefill_grouped_down", "mixed_grouped"])
def test_deterministic(name):
    _need_gpu()
    case, view, dev = staged(name)
    a = dev.run()
    b = dev.run()
    assert np.array_equal(a, b)


def test_grouped_equals_gather_permuted():
    """Grouped row r equals gather row sorted_ids[r], bit for bit (same inputs)."""
    _need_gpu()
    from staging import DeviceCase
    g = workloads.make_grouped_case(71, stream_lens=[300, 97, 211], top_k=4, n_route=24,
                                    k_in=256, n_out=512, max_rank=32, routing="zipf",
                                    n_unadapted=4, cap=200, stream_slot_values=[1, -1, 1])
    dg = DeviceCase(g, DEV)
    out_g = dg.run()
    flat = workloads.FoldCase(**{k: getattr(g, k) for k in g.__dataclass_fields__})
    flat.path = "gather"
    flat.indices = g.notes["indices_flat"]
    inv = np.empty_like(g.sorted_ids)
    inv[g.sorted_ids] = np.arange(g.sorted_ids.shape[0], dtype=g.sorted_ids.dtype)
    flat.base = g.base[inv]  # flat row i holds the base of its sorted position
    df = DeviceCase(flat, DEV)
    out_f = df.run()
    assert np.array_equal(out_g, out_f[g.sorted_ids])


def test_windows_equal_single_window():
    _need_gpu()
    case, view, dev = staged("prefill_grouped_down")
    a = dev.run(windows=[(0, case.n_rows)])
    b = dev.run()  # four windows of 8192
    assert np.array_equal(a, b)
    c = dev.run(windows=[(0, 1000), (1000, 1001), (1001, 20000), (20000, case.n_rows)])
    assert np.array_equal(a, c)


def test_scale_power_of_two_is_exact():
    """Z run: scaling every scale by 4 scales every output by 4, bit for bit."""
    _need_gpu()
    from staging import DeviceCase
    c1 = workloads.make_gather_case(72, n_seq=40, padded_n=48, top_k=4, n_route=16, k_in=320,
                                    n_out=384, max_rank=16, skip_seqs=3)
    c1.base = np.zeros_like(c1.base)
    c2 = workloads.FoldCase(**{k: getattr(c1, k) for k in c1.__dataclass_fields__})
    c2.entries = [(e, a, b, s * 4.0) for (e, a, b, s) in c1.entries]
    o1 = to_f64(DeviceCase(c1, DEV).run(), "bf16")
    o2 = to_f64(DeviceCase(c2, DEV).run(), "bf16")
    assert np.array_equal(o2, 4.0 * o1)
    assert np.any(o1 != 0)


def test_b_zero_leaves_base():
    _need_gpu()
    from staging import DeviceCase
    c = workloads.make_grouped_case(73, stream_lens=[90, 70], top_k=2, n_route=8, k_in=128,
                                    n_out=256, max_rank=16, cap=64)
    c.b_pool = np.zeros_like(c.b_pool)
    got = DeviceCase(c, DEV).run()
    assert np.array_equal(to_f64(got, "bf16"), to_f64(c.base, "bf16"))


def test_integer_inputs_bit_exact():
    """Inputs in {-1, 0, 1}, scales in {1/2, 1, 2}: every partial sum is exact
    in fp32 and bf16, so the device result equals the oracle exactly."""
    _need_gpu()
    from staging import DeviceCase
    rng = np.random.default_rng(74)
    for path in ("gather", "grouped"):
        if path == "gather":
            c = workloads.make_gather_case(75, n_seq=30, padded_n=36, top_k=3, n_route=9,
                                           k_in=96, n_out=136, max_rank=24, skip_seqs=4,
                                           wild_index_frac=0.1)
        else:
            c = workloads.make_grouped_case(76, stream_lens=[50, 61], top_k=3, n_route=9,
                                            k_in=96, n_out=136, max_rank=24, n_unadapted=2,
                                            cap=70, dup_frac=0.3)
        bits = {-1: 0xBF80, 0: 0x0000, 1: 0x3F80}

        def tern(shape):
            v = rng.integers(-1, 2, size=shape)
            return np.vectorize(lambda t: bits[int(t)])(v).astype(np.uint16)

        # two non-zeros per x row keep |h| <= 2 and every output within bf16's
        # exact-integer range
        x = np.zeros(c.x.shape, dtype=np.uint16)
        for t in range(x.shape[0]):
            cols = rng.choice(x.shape[1], size=2, replace=False)
            x[t, cols] = [bits[int(v)] for v in rng.choice([-1, 1], size=2)]
        c.x = x
        c.a_pool = tern(c.a_pool.shape)
        c.b_pool = tern(c.b_pool.shape)
        c.base = tern(c.base.shape)
        c.entries = [(e, a, b, [0.5, 1.0, 2.0][i % 3]) for i, (e, a, b, _) in enumerate(c.entries)]
        view = OracleView(c)
        ref = view.fold()
        assert np.abs(ref).max() <= 256
        got = to_f64(DeviceCase(c, DEV).run(), "bf16")
        assert np.array_equal(got, ref), path


def test_rank1_onehot_closed_form():
    """One-hot x rows and rank 1: delta = scale * A[0, i] * B[:, 0]."""
    _need_gpu()
    from staging import DeviceCase
    c = workloads.make_gather_case(77, n_seq=20, padded_n=20, top_k=2, n_route=5, k_in=64,
                                   n_out=96, max_rank=1)
    hot = np.random.default_rng(78).integers(0, 64, size=c.x.shape[0])
    x = np.zeros(c.x.shape, dtype=np.uint16)
    x[np.arange(x.shape[0]), hot] = 0x3F80
    c.x = x
    c.base = np.zeros_like(c.base)
    got = to_f64(DeviceCase(c, DEV).run(), "bf16")
    view = OracleView(c)
    for row in range(c.n_rows):
        e = int(c.indices[row])
        t = row // c.top_k
        if not (0 <= e < view.n_experts and view.a_table[e] and view.b_table[e]):
            continue
        a = to_f64(c.a_pool[view_handle(c, e)], "bf16")
        b = to_f64(c.b_pool[view_handle(c, e)], "bf16")
        want = view.scale_table[e] * a[0, hot[t]] * b[:, 0]
        assert np.allclose(got[row], want, rtol=8e-3, atol=1e-6)


def view_handle(c, e):
    h = None
    for (ee, a, _, _) in c.entries:
        if ee == e:
            h = a
    return h


SMALL = [
    # (label, builder kwargs)
    ("gather_ragged_r8", dict(kind="gather", n_seq=13, padded_n=17, top_k=3, n_route=11,
                              k_in=40, n_out=72, max_rank=8, skip_seqs=2, refuse_seqs=1,
                              wild_index_frac=0.15, n_adapted=7)),
    ("gather_r24_k72", dict(kind="gather", n_seq=50, padded_n=50, top_k=5, n_route=12,
                            k_in=72, n_out=104, max_rank=24, n_adapted=10, dup_frac=0.3)),
    ("gather_r48", dict(kind="gather", n_seq=64, padded_n=70, top_k=4, n_route=6, k_in=200,
                        n_out=136, max_rank=48, skip_seqs=5)),
    ("gather_r17_decode", dict(kind="gather", n_seq=30, padded_n=32, top_k=8, n_route=24,
                               k_in=256, n_out=200, max_rank=17, skip_seqs=2, n_adapted=20)),
    ("gather_r100", dict(kind="gather", n_seq=37, padded_n=40, top_k=2, n_route=5, k_in=264,
                         n_out=520, max_rank=100)),
    ("gather_r128", dict(kind="gather", n_seq=33, padded_n=33, top_k=3, n_route=4, k_in=128,
                         n_out=96, max_rank=128)),
    ("gather_r64_many_rows", dict(kind="gather", n_seq=700, padded_n=700, top_k=2, n_route=3,
                                  k_in=512, n_out=264, max_rank=64)),
    ("gather_topk1_one_expert", dict(kind="gather", n_seq=3000, padded_n=3000, top_k=1,
                                     n_route=1, k_in=256, n_out=128, max_rank=16,
                                     index_mode="zero", adapted=np.array([0]))),
    ("gather_slots_not_multiple", dict(kind="gather", n_seq=10, padded_n=10, top_k=4,
                                       n_route=7, k_in=64, n_out=64, max_rank=16,
                                       n_slots=37)),
    ("gather_all_skip", dict(kind="gather", n_seq=8, padded_n=8, top_k=2, n_route=4,
                             k_in=64, n_out=64, max_rank=16, skip_seqs=8)),
    ("gather_f32_r24", dict(kind="gather", n_seq=9, padded_n=11, top_k=3, n_route=6, k_in=48,
                            n_out=40, max_rank=24, dtype="f32", skip_seqs=1,
                            wild_index_frac=0.1)),
    # hidden sizes of large MoE layers: a long k (streaming kernels, k split
    # over many steps) and a wide n (many column slices)
    ("gather_k7168", dict(kind="gather", n_seq=24, padded_n=26, top_k=8, n_route=16,
                          k_in=7168, n_out=2048, max_rank=16, skip_seqs=2)),
    ("gather_n7168_r64", dict(kind="gather", n_seq=20, padded_n=20, top_k=8, n_route=12,
                              k_in=2048, n_out=7168, max_rank=64)),
    ("grouped_zipf_r32", dict(kind="grouped", stream_lens=[130, 0, 77, 300], top_k=6,
                              n_route=20, k_in=192, n_out=320, max_rank=32, routing="zipf",
                              n_unadapted=3, cap=100, stream_slot_values=[1, 1, -1, 1])),
    ("grouped_r16_wide", dict(kind="grouped", stream_lens=[257], top_k=8, n_route=40,
                              k_in=1536, n_out=1032, max_rank=16, n_unadapted=10,
                              force_unadapted=(39,), dup_frac=0.2, cap=1000)),
    ("grouped_r8_narrow", dict(kind="grouped", stream_lens=[33, 31], top_k=3, n_route=5,
                               k_in=56, n_out=24, max_rank=8, cap=7)),
    ("grouped_r64_r100", dict(kind="grouped", stream_lens=[211], top_k=2, n_route=9,
                              k_in=320, n_out=200, max_rank=100, cap=150)),
    ("grouped_r128", dict(kind="grouped", stream_lens=[100], top_k=2, n_route=3, k_in=128,
                          n_out=256, max_rank=128, cap=64)),
    ("grouped_k7168", dict(kind="grouped", stream_lens=[200, 90], top_k=8, n_route=20,
                           k_in=7168, n_out=1024, max_rank=32, cap=1000)),
    ("grouped_n7168", dict(kind="grouped", stream_lens=[150], top_k=6, n_route=16, k_in=512,
                           n_out=7168, max_rank=16, cap=400)),
    ("grouped_f32", dict(kind="grouped", stream_lens=[20, 9], top_k=3, n_route=7, k_in=40,
                         n_out=48, max_rank=12, dtype="f32", n_unadapted=2, cap=30)),
]


def build_small(label, kw):
    kw = dict(kw)
    kind = kw.pop("kind")
    seed = 1000 + sum(map(ord, label))
    if kind == "gather":
        return workloads.make_gather_case(seed, name=label, **kw)
    return workloads.make_grouped_case(seed, name=label, **kw)


@pytest.mark.parametrize("label,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(label, kw):
    _need_gpu()
    from staging import DeviceCase
    c = build_small(label, kw)
    view = OracleView(c)
    dev = DeviceCase(c, DEV)
    check(view, dev.run(), c.base, f"{label} R")
    zero = np.zeros_like(c.base)
    if view.live_rows().any():
        check(view, dev.run(zero), zero, f"{label} Z")
    live = view.live_rows()
    base = c.base.copy()
    put_sentinel(base, ~live, c.dtype)
    got = dev.run(base)
    assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))


GROUPED_SMALL = [s for s in SMALL if s[1]["kind"] == "grouped"]


@pytest.mark.parametrize("label", ["prefill_grouped_down", "mixed_grouped"] + [s[0] for s in GROUPED_SMALL])
def test_grouped_two_kernel_equals_one_kernel(label):
    """The workspace (shrink, then expand) form and the one-kernel form of the
    grouped fold give the same bits, and the one-kernel form passes the
    oracle bar on its own (the other tests run the two-kernel form)."""
    _need_gpu()
    from staging import DeviceCase
    if label in workloads.WORKLOADS:
        case, view, dev = staged(label)
    else:
        case = build_small(label, dict(SMALL)[label])
        view, dev = OracleView(case), DeviceCase(case, DEV)
    one = dev.run(two_kernel=False)
    check(view, one, case.base, f"{label} one-kernel")
    two = dev.run(two_kernel=True)
    assert np.array_equal(one.view(np.uint8), two.view(np.uint8))


@pytest.mark.parametrize("label", ["prefill_grouped_down", "mixed_grouped"] + [s[0] for s in GROUPED_SMALL])
def test_grouped_launch_shapes_give_the_same_bits(label, overrides):
    """Shrink tiles of 16, 32 or 64 rows and expand waves of 16 or 32 rows
    (MLORA_SHRINK_MB / MLORA_EXPAND_MB) change which workgroup computes a row,
    not how: every shape gives the bits of the default per-window call, and
    every first-shrink tile of the all-windows call the bits of its default."""
    _need_gpu()
    from staging import DeviceCase
    if label in workloads.WORKLOADS:
        case, view, dev = staged(label)
    else:
        case = build_small(label, dict(SMALL)[label])
        view, dev = OracleView(case), DeviceCase(case, DEV)
    ref = dev.run(two_kernel=True, pipelined=False)
    for smb, emb in [("1", "1"), ("2", "2"), ("4", "1"), ("1", "2")]:
        overrides.set("MLORA_SHRINK_MB", smb)
        overrides.set("MLORA_EXPAND_MB", emb)
        got = dev.run(two_kernel=True, pipelined=False)
        assert np.array_equal(ref.view(np.uint8), got.view(np.uint8)), (smb, emb)
    # the all-windows call's first shrink runs alone and takes the shrink tile
    # override too
    overrides.delete("MLORA_EXPAND_MB")
    overrides.delete("MLORA_SHRINK_MB")
    pipe_ref = dev.run(two_kernel=True, pipelined=True)
    for smb in ("1", "2"):
        overrides.set("MLORA_SHRINK_MB", smb)
        got = dev.run(two_kernel=True, pipelined=True)
        assert np.array_equal(pipe_ref.view(np.uint8), got.view(np.uint8)), ("first shrink", smb)


GATHER_SMALL = [s[0] for s in SMALL if s[1]["kind"] == "gather" and s[1].get("dtype") != "f32"]


@pytest.mark.parametrize("label", ["gateup_gather", "router_gather"] + GATHER_SMALL)
def test_gather_one_kernel_form(label):
    """The gather fold without a workspace (one kernel) passes the oracle bar;
    the other tests give it a workspace, which large calls use for the
    two-kernel form."""
    _need_gpu()
    from staging import DeviceCase
    if label in workloads.WORKLOADS:
        case, view, dev = staged(label)
    else:
        case = build_small(label, dict(SMALL)[label])
        view, dev = OracleView(case), DeviceCase(case, DEV)
    check(view, dev.run(two_kernel=False), case.base, f"{label} one-kernel")
    zero = np.zeros_like(case.base)
    if view.live_rows().any():
        check(view, dev.run(zero, two_kernel=False), zero, f"{label} one-kernel Z")


TWO_GATHER = ["gather_r24_k72", "gather_r48", "gather_r100", "gather_r128",
              "gather_r64_many_rows", "gather_topk1_one_expert", "gather_slots_not_multiple",
              "gather_all_skip", "gather_k1000_r100", "gather_k2048_r64_skew"]


def _two_gather_case(label):
    if label == "gather_k1000_r100":
        return workloads.make_gather_case(83, n_seq=60, padded_n=64, top_k=4, n_route=20,
                                          k_in=1000, n_out=392, max_rank=100, n_adapted=15,
                                          skip_seqs=4, name=label)
    if label == "gather_k2048_r64_skew":
        return workloads.make_gather_case(84, n_seq=300, padded_n=300, top_k=2, n_route=3,
                                          k_in=2048, n_out=264, max_rank=64, name=label)
    return build_small(label, dict(SMALL)[label])


@pytest.mark.parametrize("label", TWO_GATHER)
def test_gather_two_kernel_form(label, overrides):
    """The two-kernel gather (k-split shrink into the workspace, then expand),
    forced on: oracle bar on a random and a zero base, untouched rows bit
    for bit. k_in 1000 and 2048 split into 2 and 4 k ranges."""
    _need_gpu()
    from staging import DeviceCase
    overrides.set("MLORA_GATHER_TWO", "1")
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    case = _two_gather_case(label)
    view, dev = OracleView(case), DeviceCase(case, DEV)
    check(view, dev.run(two_kernel=True), case.base, f"{label} two-kernel")
    zero = np.zeros_like(case.base)
    if view.live_rows().any():
        check(view, dev.run(zero, two_kernel=True), zero, f"{label} two-kernel Z")
    live = view.live_rows()
    base = case.base.copy()
    put_sentinel(base, ~live, case.dtype)
    got = dev.run(base, two_kernel=True)
    assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))


@pytest.mark.parametrize("min_rows", [None, "1"], ids=["launch16k", "launch1win"])
@pytest.mark.parametrize("label", ["prefill_grouped_down", "mixed_grouped"] + [s[0] for s in GROUPED_SMALL])
def test_grouped_all_windows_pipelined_equals_per_window(label, min_rows, overrides):
    """mlora_grouped_down_all (launch l + 1's windows shrunk in the launch that
    expands launch l's) equals one mlora_grouped_down call per window, bit for
    bit, with launches of >= 16384 rows (the default) and of one window."""
    _need_gpu()
    if min_rows:
        overrides.set("MLORA_ALL_MIN_ROWS", min_rows)
    from staging import DeviceCase
    if label in workloads.WORKLOADS:
        case, view, dev = staged(label)
    else:
        case = build_small(label, dict(SMALL)[label])
        view, dev = OracleView(case), DeviceCase(case, DEV)
    per_window = dev.run(two_kernel=True, pipelined=False)
    pipelined = dev.run(two_kernel=True, pipelined=True)
    assert np.array_equal(per_window.view(np.uint8), pipelined.view(np.uint8))


@pytest.mark.parametrize("min_rows", ["1", "120", None])
def test_grouped_all_many_small_windows(min_rows, overrides):
    """Many windows (cap 40 over 1203 rows), launched one window at a time,
    three windows at a time, or all at once: both workspace slots alternate."""
    _need_gpu()
    if min_rows:
        overrides.set("MLORA_ALL_MIN_ROWS", min_rows)
    from staging import DeviceCase
    case = workloads.make_grouped_case(95, stream_lens=[200, 101], top_k=4, n_route=9,
                                       k_in=320, n_out=264, max_rank=24, routing="zipf",
                                       n_unadapted=2, cap=40, stream_slot_values=[1, 1])
    view, dev = OracleView(case), DeviceCase(case, DEV)
    assert len(dev.windows) > 20
    check(view, dev.run(two_kernel=True, pipelined=True), case.base, "cap40 pipelined")
    assert np.array_equal(dev.run(two_kernel=True, pipelined=True).view(np.uint8),
                          dev.run(two_kernel=True, pipelined=False).view(np.uint8))


UNNAMED = [
    ("bf16_r32", dict(stream_lens=[300, 211, 97], top_k=4, n_route=24, k_in=320, n_out=272,
                      max_rank=32, routing="zipf", n_unadapted=4, cap=256)),
    ("bf16_r16", dict(stream_lens=[150, 77], top_k=8, n_route=40, k_in=256, n_out=520,
                      max_rank=16, n_unadapted=9, cap=300)),
    ("bf16_r48", dict(stream_lens=[64, 65], top_k=2, n_route=9, k_in=136, n_out=96,
                      max_rank=48, n_unadapted=2, cap=100)),
    ("f32", dict(stream_lens=[31, 20], top_k=4, n_route=12, k_in=64, n_out=40, max_rank=8,
                 dtype="f32", n_unadapted=2, cap=64)),
]


@pytest.mark.parametrize("form", ["one_kernel", "two_kernel", "pipelined", "pipelined_1win"])
@pytest.mark.parametrize("label,kw", UNNAMED, ids=[u[0] for u in UNNAMED])
def test_grouped_unnamed_rows(label, kw, form, overrides):
    """Sorted rows that name no token (id -1, an id at/after n_tokens * top_k)
    inside spans, and rows before the first span and after the last one, fold
    nothing in every grouped form: they keep a signalling-NaN sentinel bit
    for bit, and every other row meets the bound."""
    from staging import DeviceCase
    _need_gpu()
    c = workloads.make_grouped_case(71, **kw)
    u = workloads.with_unnamed_rows(c, 71, lead=37, tail=29, bad_frac=0.15)
    assert (u.sorted_ids < 0).any() and (u.sorted_ids >= u.n_tokens * u.top_k).any()
    view, dev = OracleView(u), DeviceCase(u, DEV)
    if form == "pipelined_1win":
        overrides.set("MLORA_ALL_MIN_ROWS", 1)
    two = form != "one_kernel"
    pipe = form.startswith("pipelined")
    live = view.live_rows()
    assert (~live).sum() > 66
    base = u.base.copy()
    put_sentinel(base, ~live, u.dtype)
    got = dev.run(base, two_kernel=two, pipelined=pipe)
    assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))
    check(view, dev.run(two_kernel=two, pipelined=pipe), u.base, f"{label} unnamed {form}")


@pytest.mark.parametrize("label", ["prefill_grouped_down", "mixed_grouped", "unnamed"])
@pytest.mark.parametrize("two", [True, False], ids=["two_kernel", "one_kernel"])
def test_host_loop_baseline_equals_device_routed(label, two):
    """mlora_apply_expert_lora_sorted (spans copied to the host, one launch per
    adapted expert) gives the bits of the device-routed fold over every row."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch
    _need_gpu()
    if label == "unnamed":
        case = workloads.with_unnamed_rows(
            workloads.make_grouped_case(72, **UNNAMED[0][1]), 72, lead=11, tail=5,
            bad_frac=0.1)
    else:
        case = workloads.WORKLOADS[label]()
    dev = DeviceCase(case, DEV)
    want = dev.run(windows=[(0, case.n_rows)], two_kernel=two)
    off_h = dev.offsets.cpu().numpy()
    at, bt, _, _ = dev.tables_host
    spans = np.diff(off_h.astype(np.int64))
    ws = None
    if two:
        ws = torch.empty(max(256, ml.mlora_grouped_down_workspace_bytes(0, int(spans.max()),
                                                                        case.max_rank)),
                         dtype=torch.uint8, device=DEV)
    out = dev.base0.clone()
    ml.mlora_apply_expert_lora_sorted(dev.route, dev.x, out, dev.offsets, off_h, at, bt,
                                      dev.sorted_ids, dev.row_adapter, case.top_k, workspace=ws)
    torch.cuda.synchronize()
    got = from_torch(out)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


def test_grouped_workspace_reused_across_windows_and_calls():
    """One workspace serves successive windows and calls; stale contents from a
    larger call never leak into a smaller one."""
    _need_gpu()
    from staging import DeviceCase
    big = workloads.make_grouped_case(91, stream_lens=[300, 211], top_k=4, n_route=12,
                                      k_in=256, n_out=384, max_rank=32, routing="zipf",
                                      n_unadapted=2, cap=256)
    small = workloads.make_grouped_case(92, stream_lens=[40], top_k=2, n_route=12,
                                        k_in=256, n_out=384, max_rank=32, n_unadapted=5,
                                        cap=64, stream_slot_values=[1])
    db, ds = DeviceCase(big, DEV), DeviceCase(small, DEV)
    ds._ws = db.workspace_for(db.windows)  # shared
    for _ in range(2):
        got_b = db.run()
        ds._ws = db._ws
        got_s = ds.run()
        check(OracleView(big), got_b, big.base, "big")
        check(OracleView(small), got_s, small.base, "small")


@pytest.mark.parametrize("label", ["decode_down_gather", "gather_r24_k72", "gather_slots_not_multiple",
                                   "gather_r16_ns4", "gather_ragged_r8", "gather_r17_decode"])
def test_resident_weights_path_equals_streaming_path(label, overrides):
    """The decode path that holds a wave's weights in registers and the
    streaming path fold in the same order: outputs equal bit for bit, and the
    resident one passes the oracle bar on its own."""
    _need_gpu()
    from staging import DeviceCase
    if label == "decode_down_gather":
        case, view, dev = staged(label)
    elif label == "gather_r16_ns4":
        case = workloads.make_gather_case(77, n_seq=40, padded_n=48, top_k=6, n_route=30,
                                          k_in=1000, n_out=1000, max_rank=16, n_adapted=25,
                                          skip_seqs=3, name=label)
        view, dev = OracleView(case), None
    else:
        case = build_small(label, dict(SMALL)[label])
        view, dev = OracleView(case), None
    dev = dev or DeviceCase(case, DEV)
    if label == "gather_r16_ns4":
        overrides.set("MLORA_GATHER_NS", "4")
    overrides.set("MLORA_GATHER_RESIDENT", "1")
    res = dev.run()
    check(view, res, case.base, f"{label} resident")
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    stream = dev.run(two_kernel=False)
    assert np.array_equal(res.view(np.uint8), stream.view(np.uint8))


@pytest.mark.parametrize("n_seq,form", [(64, "one"), (96, "one"), (128, "two")])
def test_gather_planner_default_form(n_seq, form, overrides):
    """With a workspace, a gather whose experts average at most 6 rows (k_in
    2048, rank 16) runs as one kernel (the decode kernel's wide form, whose
    bits are the streaming kernel's), from 7 rows on as the k-split pair. The
    two forms add the k ranges in different orders, so the default call's bits
    show which one ran; both pass the oracle bar."""
    _need_gpu()
    from staging import DeviceCase
    case = workloads.make_gather_case(90 + n_seq, n_seq=n_seq, padded_n=n_seq, top_k=8,
                                      n_route=128, k_in=2048, n_out=768, max_rank=16,
                                      name=f"planner_{n_seq}")
    view, dev = OracleView(case), DeviceCase(case, DEV)
    got = dev.run()
    check(view, got, case.base, f"{case.name} default")
    forced = {}
    overrides.set("MLORA_GATHER_RESIDENT", "0")  # the one-kernel form is the streaming one
    for f, two in (("one", "0"), ("two", "1")):
        overrides.set("MLORA_GATHER_TWO", two)
        forced[f] = dev.run()
    overrides.delete("MLORA_GATHER_TWO")
    overrides.delete("MLORA_GATHER_RESIDENT")
    assert not np.array_equal(forced["one"], forced["two"])
    assert np.array_equal(got.view(np.uint8), forced[form].view(np.uint8))


def test_guard_bands_untouched():
    """Fold into a slice of a larger buffer: the bytes around it stay as they were."""
    _need_gpu()
    from staging import DeviceCase, from_torch, to_torch
    c = workloads.make_grouped_case(79, stream_lens=[120], top_k=4, n_route=10, k_in=128,
                                    n_out=256, max_rank=32, cap=100)
    dev = DeviceCase(c, DEV)
    pad = 4096
    flat = np.random.default_rng(80).integers(0, 1 << 16, size=c.base.size + 2 * pad,
                                              dtype=np.uint64).astype(np.uint16)
    flat[pad:pad + c.base.size] = c.base.reshape(-1)
    buf = to_torch(flat, "bf16", DEV)
    view = buf[pad:pad + c.base.size].view(c.base.shape)
    dev.fold(view)
    torch.cuda.synchronize()
    after = from_torch(buf)
    assert np.array_equal(after[:pad], flat[:pad])
    assert np.array_equal(after[pad + c.base.size:], flat[pad + c.base.size:])
    check(OracleView(c), after[pad:pad + c.base.size].reshape(c.base.shape), c.base, "guard")


def test_empty_calls_enqueue_nothing():
    _need_gpu()
    from staging import DeviceCase
    c = workloads.make_grouped_case(81, stream_lens=[40], top_k=2, n_route=4, k_in=64,
                                    n_out=64, max_rank=16, cap=64)
    dev = DeviceCase(c, DEV)
    got = dev.run(windows=[(10, 10), (80, 80)])
    assert np.array_equal(got, c.base)


def test_graph_replay_reads_routing_on_device():
    """A fold captured in a HIP graph and replayed matches the eager fold, and a
    replay after the routing (indices, map) and table cells are rewritten in
    place uses the new contents: the host never reads routing data."""
    _need_gpu()
    from staging import DeviceCase, from_torch, to_torch
    c = workloads.make_gather_case(82, n_seq=48, padded_n=56, top_k=4, n_route=16, k_in=256,
                                   n_out=320, max_rank=16, n_adapted=12, skip_seqs=4)
    dev = DeviceCase(c, DEV)
    pristine = to_torch(c.base, "bf16", DEV)
    base = pristine.clone()
    eager1 = dev.run()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dev.fold(base)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        base.copy_(pristine)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_torch(base), eager1)
    # new routing, new map and one table cell cleared, written in place
    rng = np.random.default_rng(83)
    new_idx = rng.integers(0, 16, size=c.indices.shape, dtype=np.int64).astype(np.int32)
    new_map = np.where(rng.random(dev.row_adapter.numel()) < 0.3, -1, 1).astype(np.int32)
    dev.indices.copy_(torch.from_numpy(new_idx))
    dev.row_adapter.copy_(torch.from_numpy(new_map))
    live_e = int(np.flatnonzero(dev.tables_host[0])[0])
    dev.a_table[live_e] = 0
    base.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    c2 = workloads.FoldCase(**{k: getattr(c, k) for k in c.__dataclass_fields__})
    c2.indices = new_idx
    view = OracleView(c2)
    view.row_adapter = new_map
    view.a_table = list(view.a_table)
    view.a_table[live_e] = 0
    check(view, from_torch(base), c.base, "graph replay, new routing")


@pytest.mark.parametrize("form", ["grouped_all", "grouped_all_per_window",
                                  "grouped_all_block_order", "grouped_window", "gather_two"])
def test_graph_replay_workspace_forms(form, overrides):
    """The workspace forms captured in a HIP graph: every replay (with eager
    work and syncs between) equals the eager fold bit for bit, and a replay
    after the map and one table cell are rewritten in place folds by the new
    contents."""
    _need_gpu()
    from staging import DeviceCase, from_torch, to_torch
    if form == "gather_two":
        overrides.set("MLORA_GATHER_TWO", "1")
        overrides.set("MLORA_GATHER_RESIDENT", "0")
        c = workloads.make_gather_case(86, n_seq=40, padded_n=48, top_k=4, n_route=10,
                                       k_in=1024, n_out=256, max_rank=32, n_adapted=8,
                                       skip_seqs=3)
        dev = DeviceCase(c, DEV)
    else:
        c = workloads.make_grouped_case(87, stream_lens=[150, 90, 61], top_k=4, n_route=12,
                                        k_in=256, n_out=320, max_rank=32, routing="zipf",
                                        n_unadapted=2, cap=300, stream_slot_values=[1, 1, 1])
        if form == "grouped_all_per_window":
            # one window per launch: the pipe kernel runs inside the graph
            overrides.set("MLORA_ALL_MIN_ROWS", "1")
        if form == "grouped_all_block_order":
            # expand units in block order (this shape's plan takes XCD shares)
            overrides.set("MLORA_ALL_MIN_ROWS", "1")
            overrides.set("MLORA_EXPAND_XCD", "0")
        dev = DeviceCase(c, DEV, pipelined=form.startswith("grouped_all"))
        assert len(dev.windows) > 1
    dev.workspace_for(getattr(dev, "windows", None))   # allocated before capture
    pristine = to_torch(c.base, "bf16", DEV)
    base = pristine.clone()
    eager = dev.run()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dev.fold(base)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        base.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_torch(base).view(np.uint8), eager.view(np.uint8))
    rng = np.random.default_rng(88)
    new_map = np.where(rng.random(dev.row_adapter.numel()) < 0.3, -1, 1).astype(np.int32)
    dev.row_adapter.copy_(torch.from_numpy(new_map))
    live_e = int(np.flatnonzero(dev.tables_host[1])[0])
    dev.b_table[live_e] = 0
    base.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    view = OracleView(c)
    view.row_adapter = new_map
    view.b_table = list(view.b_table)
    view.b_table[live_e] = 0
    check(view, from_torch(base), c.base, f"{form} graph replay, new map and table")



@pytest.mark.parametrize("label", ["router_gather", "router_skips_wild", "router_r32_k768",
                                   "router_rows_not_multiple", "router_null_cell"])
def test_dense_slices_equal_compacting_kernel(label, overrides):
    """A one-entry route runs as dense slices (rows taken in place, no routing
    compaction); the compacting kernel folds every row in the same order, so
    the outputs are equal bit for bit, skipped and wild rows untouched, and the
    dense form passes the oracle bar on its own."""
    _need_gpu()
    from staging import DeviceCase
    if label == "router_gather":
        case, view, dev = staged(label)
    else:
        kw = dict(n_seq=6, padded_n=300, top_k=1, n_route=1, k_in=2048, n_out=160, max_rank=16,
                  adapted=np.array([0]), index_mode="zero", name=label)
        if label == "router_skips_wild":
            kw.update(n_seq=40, padded_n=333, skip_seqs=5, wild_index_frac=0.1, n_slots=333)
        elif label == "router_r32_k768":
            kw.update(k_in=768, max_rank=32, n_out=96, padded_n=250)
        elif label == "router_rows_not_multiple":
            kw.update(padded_n=37, k_in=1000, max_rank=12, n_out=72)
        case = workloads.make_gather_case(314, **kw)
        if label == "router_null_cell":
            # the one cell is packed without matrices: nothing folds
            case.entries = [(0, workloads.NULL_HANDLE, workloads.NULL_HANDLE, 0.0)]
        view, dev = OracleView(case), DeviceCase(case, DEV)
    dense = dev.run()
    check(view, dense, case.base, f"{label} dense")
    overrides.set("MLORA_GATHER_DENSE", "0")
    compact = dev.run()
    assert np.array_equal(dense.view(np.uint8), compact.view(np.uint8))


def test_graph_replay_dense_one_entry_route():
    """The dense-slice kernel (a one-entry route) captured in a HIP graph:
    replays match the eager fold, and replays after the map, then the table
    cell, are rewritten in place follow the new contents."""
    _need_gpu()
    from staging import DeviceCase, from_torch, to_torch
    c = workloads.make_gather_case(84, n_seq=1, padded_n=300, top_k=1, n_route=1, k_in=1024,
                                   n_out=96, max_rank=16, adapted=np.array([0]),
                                   index_mode="zero", name="graph_dense")
    dev = DeviceCase(c, DEV)
    pristine = to_torch(c.base, "bf16", DEV)
    base = pristine.clone()
    eager = dev.run()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dev.fold(base)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        base.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_torch(base), eager)
    # a new map: about a third of the token rows skip
    rng = np.random.default_rng(85)
    new_map = np.where(rng.random(dev.row_adapter.numel()) < 0.35, -1, 1).astype(np.int32)
    dev.row_adapter.copy_(torch.from_numpy(new_map))
    base.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    view = OracleView(c)
    view.row_adapter = new_map
    check(view, from_torch(base), c.base, "graph replay dense, new map")
    # the cell cleared: nothing folds
    dev.b_table[0] = 0
    base.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(from_torch(base), c.base)


# slice lengths on both sides of each routing-round count of the decode
# kernel (256 rows a round; 1, 2, 3, 4 or 8 rounds) and of a second row slice
# (2048 rows a slice)
ROUND_EDGES = [200, 256, 257, 512, 600, 768, 769, 1024, 1100, 2048, 2056]


@pytest.mark.parametrize("n_slots", ROUND_EDGES)
def test_decode_kernel_routing_rounds(n_slots, overrides):
    """The decode kernel at every routing-round count and across a second row
    slice: the oracle bound, and the bits of the streaming kernel."""
    _need_gpu()
    from staging import DeviceCase
    top_k = 8
    n_seq = -(-n_slots // top_k)
    case = workloads.make_gather_case(3000 + n_slots, n_seq=n_seq, padded_n=n_seq, top_k=top_k,
                                      n_route=128, k_in=256, n_out=512, max_rank=16,
                                      n_adapted=100, skip_seqs=max(1, n_seq // 16),
                                      n_slots=n_slots, name=f"rounds_{n_slots}")
    view, dev = OracleView(case), DeviceCase(case, DEV)
    overrides.set("MLORA_GATHER_RESIDENT", "1")
    res = dev.run(two_kernel=False)
    check(view, res, case.base, f"rounds_{n_slots} decode kernel")
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    stream = dev.run(two_kernel=False)
    assert np.array_equal(res.view(np.uint16), stream.view(np.uint16))


@pytest.mark.parametrize("k_in", [8, 760, 768, 776, 1016, 1024])
def test_decode_kernel_k_steps(k_in, overrides):
    """The decode kernel on both sides of its k-step counts (6 steps a wave up
    to k_in 768, 8 up to 1024): the oracle bound, and the bits of the
    streaming kernel."""
    _need_gpu()
    from staging import DeviceCase
    case = workloads.make_gather_case(3100 + k_in, n_seq=40, padded_n=44, top_k=8, n_route=64,
                                      k_in=k_in, n_out=1032, max_rank=16, n_adapted=50,
                                      skip_seqs=3, name=f"ksteps_{k_in}")
    view, dev = OracleView(case), DeviceCase(case, DEV)
    overrides.set("MLORA_GATHER_RESIDENT", "1")
    res = dev.run(two_kernel=False)
    check(view, res, case.base, f"ksteps_{k_in} decode kernel")
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    stream = dev.run(two_kernel=False)
    assert np.array_equal(res.view(np.uint16), stream.view(np.uint16))
