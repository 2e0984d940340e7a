"""GPU parity of the per-layer projection set (mlora_gather_bgmv_set, one
launch for several gather calls), through the C ABI.

A decode layer's folds as a set: a one-entry router route over the tokens,
gate and up over the (token, slot) rows writing the two halves of one fused
[rows, 2 * n_out] output (row stride 2 * n_out), and down reading slot-major
x (one x row per flat row). Every projection of a set must come out exactly
as the same call alone (bit for bit), meet the oracle bound, and leave every
element outside its rows and columns untouched.
"""
from __future__ import annotations

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


def layer_cases(seed=100):
    """A decode layer's router, gate, up and slot-major down folds at small
    sizes (24 sequences x top-4 over 40 experts, hidden 512, inter 384)."""
    return workloads.decode_layer_cases(seed=seed, n_seq=24, padded_n=32, top_k=4, n_route=40,
                                        n_adapted=34, skip_seqs=3, hidden=512, inter=384)


def oracle_fold(case, base):
    import oracle
    view = OracleView(case)
    x_rows = case.notes.get("x_rows", "token")
    ref = oracle.fold_gather(view.x, view.a_table, view.b_table, view.scale_table, view.mats,
                             to_f64(base, case.dtype), case.indices, view.row_adapter,
                             case.top_k, x_rows=x_rows)
    return view, ref


def test_layer_set_equals_calls_alone_and_the_oracle():
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch, to_torch
    _need_gpu()
    router, gate, up, down = layer_cases()
    devs = {c.name: DeviceCase(c, DEV) for c in (router, gate, up, down)}
    inter = gate.n_out
    # fused gate/up output with a 16-column guard band after each half's row
    guard = 16
    fused0 = np.full((gate.n_rows, 2 * inter + guard), 0x7F81, dtype=np.uint16)
    fused0[:, :inter] = gate.base
    fused0[:, inter:2 * inter] = up.base
    fused = to_torch(fused0, "bf16", DEV)
    outs = {"router": devs["router"].base0.clone(), "down": devs["down"].base0.clone()}
    projs = [
        ml.make_projection(devs["router"].route, devs["router"].x, outs["router"],
                           devs["router"].indices, devs["router"].row_adapter, 1),
        ml.make_projection(devs["gate"].route, devs["gate"].x, fused[:, :inter],
                           devs["gate"].indices, devs["gate"].row_adapter, gate.top_k),
        ml.make_projection(devs["up"].route, devs["up"].x, fused[:, inter:2 * inter],
                           devs["up"].indices, devs["up"].row_adapter, up.top_k),
        ml.make_projection(devs["down"].route, devs["down"].x, outs["down"],
                           devs["down"].indices, devs["down"].row_adapter, down.top_k,
                           x_by_row=True),
    ]
    ml.mlora_gather_bgmv_set(projs)
    torch.cuda.synchronize()
    got_f = from_torch(fused)
    got = {"router": from_torch(outs["router"]), "gate": got_f[:, :inter],
           "up": got_f[:, inter:2 * inter], "down": from_torch(outs["down"])}
    # the guard band after the two halves is untouched
    assert np.all(got_f[:, 2 * inter:] == 0x7F81)
    for c in (router, gate, up):
        alone = devs[c.name].run(two_kernel=False)
        assert np.array_equal(got[c.name].view(np.uint16), alone.view(np.uint16)), c.name
    # one projection alone through the set entry equals the plain call
    solo = devs["gate"].base0.clone()
    ml.mlora_gather_bgmv_set([ml.make_projection(devs["gate"].route, devs["gate"].x, solo,
                                                 devs["gate"].indices,
                                                 devs["gate"].row_adapter, gate.top_k)])
    torch.cuda.synchronize()
    assert np.array_equal(from_torch(solo), got["gate"])
    for c in (router, gate, up, down):
        view, ref = oracle_fold(c, c.base)
        rel, mx, ex = parity_figures(view, to_f64(got[c.name], "bf16"), ref, f"set {c.name}")
        print(f"set {c.name}: rel_l2={rel:.3e} max_abs={mx:.3e} max_abs/limit={ex:.3f}",
              flush=True)
        assert rel <= REL_L2_TOL and ex <= 1.0, c.name
        live = view.live_rows()
        assert np.array_equal(got[c.name][~live], c.base[~live]), c.name


def test_slot_major_down_rows_and_untouched_rows():
    """Slot-major x: every row folds its own x row; rows the fold skips keep
    a signalling-NaN sentinel bit for bit; and x rows that repeat each
    token's row top_k times fold exactly as the token-major call."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch, to_torch
    _need_gpu()
    _, gate, _, down = layer_cases(seed=120)
    dev = DeviceCase(down, DEV)
    view, _ = oracle_fold(down, down.base)
    live = view.live_rows()
    base = down.base.copy()
    base.view(np.uint16)[~live] = 0x7F81
    out = to_torch(base, "bf16", DEV)
    ml.mlora_gather_bgmv_set([ml.make_projection(dev.route, dev.x, out, dev.indices,
                                                 dev.row_adapter, down.top_k, x_by_row=True)])
    torch.cuda.synchronize()
    got = from_torch(out)
    assert np.array_equal(got[~live], base[~live])
    # repeated token rows == token-major
    g = DeviceCase(gate, DEV)
    want = g.run(two_kernel=False)
    x_rep = g.x.repeat_interleave(gate.top_k, dim=0)[: gate.n_rows].contiguous()
    out2 = g.base0.clone()
    ml.mlora_gather_bgmv_set([ml.make_projection(g.route, x_rep, out2, g.indices,
                                                 g.row_adapter, gate.top_k, x_by_row=True)])
    torch.cuda.synchronize()
    assert np.array_equal(from_torch(out2), want)


@pytest.mark.parametrize("shape", ["resident", "streaming_r32", "mixed_empty"])
def test_set_shapes(shape):
    """Sets that run the resident decode kernel (k_in <= 1024, rank 16), the
    streaming one (ranks 32, 24 and 20: two rank blocks each), and a set with
    an empty projection (no rows): each member equals its call alone."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch
    _need_gpu()
    if shape == "resident":
        cases = [workloads.decode_down_gather(),
                 workloads.make_gather_case(130, n_seq=40, padded_n=48, top_k=8, n_route=64,
                                            k_in=640, n_out=1024, max_rank=16, n_adapted=50,
                                            skip_seqs=4)]
    elif shape == "streaming_r32":
        cases = [workloads.make_gather_case(131 + i, n_seq=100, padded_n=100, top_k=4,
                                            n_route=32, k_in=1536 + 256 * i, n_out=264,
                                            max_rank=(32, 24, 20)[i], n_adapted=30)
                 for i in range(3)]
    else:
        cases = [workloads.make_gather_case(140, n_seq=30, padded_n=30, top_k=2, n_route=12,
                                            k_in=256, n_out=200, max_rank=16, n_adapted=10),
                 workloads.make_gather_case(141, n_seq=0, padded_n=0, top_k=2, n_route=12,
                                            k_in=256, n_out=200, max_rank=16, n_adapted=10,
                                            n_slots=0),
                 workloads.make_gather_case(142, n_seq=10, padded_n=10, top_k=2, n_route=12,
                                            k_in=256, n_out=200, max_rank=16, n_adapted=10)]
    devs = [DeviceCase(c, DEV) for c in cases]
    outs = [d.base0.clone() for d in devs]
    projs = [ml.make_projection(d.route, d.x, o, d.indices, d.row_adapter, c.top_k)
             for c, d, o in zip(cases, devs, outs)]
    ml.mlora_gather_bgmv_set(projs)
    torch.cuda.synchronize()
    for c, d, o in zip(cases, devs, outs):
        if c.n_rows == 0:
            continue
        alone = d.run(two_kernel=False)
        assert np.array_equal(from_torch(o).view(np.uint16), alone.view(np.uint16)), c.name


@pytest.mark.parametrize("x_by_row", [False, True])
def test_one_entry_route_dense_slices_with_strides(x_by_row, overrides):
    """A one-entry route (top_k 3, so token and flat row differ) as a
    one-member set with strided x and base_out: the dense-slice kernel it
    runs on equals the compacting kernel bit for bit, meets the oracle bound
    (slot-major x when x_by_row), and leaves the guard columns untouched."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch, to_torch
    _need_gpu()
    case = workloads.make_gather_case(271, n_seq=30, padded_n=37, top_k=3, n_route=1, k_in=520,
                                      n_out=200, max_rank=16, adapted=np.array([0]),
                                      index_mode="zero", skip_seqs=4, name="one_entry_strided")
    if x_by_row:
        rng = np.random.default_rng([271, 9])
        case.x = workloads._values(rng, (case.n_rows, case.k_in), 1.0, "bf16")
        case.n_tokens = case.n_rows
        case.notes["x_rows"] = "row"
    dev = DeviceCase(case, DEV)
    gx, gout = 24, 40  # extra columns after each x / base_out row
    x_wide = np.zeros((case.x.shape[0], case.k_in + gx), dtype=np.uint16)
    x_wide[:, :case.k_in] = case.x
    x_wide[:, case.k_in:] = 0x7FC1  # NaN columns no fold may read
    xt = to_torch(x_wide, "bf16", DEV)
    outs = {}
    for dense in ("1", "0"):
        overrides.set("MLORA_GATHER_DENSE", dense)
        out0 = np.full((case.n_rows, case.n_out + gout), 0x7F81, dtype=np.uint16)
        out0[:, :case.n_out] = case.base
        out = to_torch(out0, "bf16", DEV)
        proj = ml.make_projection(dev.route, xt[:, :case.k_in], out[:, :case.n_out], dev.indices,
                                  dev.row_adapter, case.top_k, x_by_row=x_by_row)
        ml.mlora_gather_bgmv_set([proj])
        torch.cuda.synchronize()
        outs[dense] = from_torch(out)
    got = outs["1"]
    assert np.array_equal(got.view(np.uint8), outs["0"].view(np.uint8))
    assert np.all(got[:, case.n_out:] == 0x7F81)
    view, ref = oracle_fold(case, case.base)
    g = to_f64(got[:, :case.n_out], "bf16")
    rel, mx, ex = parity_figures(view, g, ref, "one_entry_strided")
    assert rel <= REL_L2_TOL and ex <= 1.0, (rel, mx, ex)
    live = view.live_rows()
    assert np.array_equal(got[~live, :case.n_out], case.base[~live])


@pytest.mark.parametrize("k_ins,rank", [((512, 768), 16), ((904, 1024), 16),
                                        ((1536, 2048), 16), ((640, 1024), 32)],
                         ids=["ks6", "ks8", "ks16_one_rank_block", "ks8_two_rank_blocks"])
def test_set_through_decode_kernel_equals_streaming_set(k_ins, rank, overrides):
    """Sets whose members fit the decode kernel's registers run through its
    body (6, 8 or, for one rank block, 16 k steps a wave): the oracle bound
    on every member, and the bits of the streaming set kernel
    (MLORA_GATHER_RESIDENT=0)."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch
    from tests.test_gpu_fold import check
    _need_gpu()
    cases = [workloads.make_gather_case(150 + i + k, n_seq=40, padded_n=44, top_k=8, n_route=64,
                                        k_in=k, n_out=(768, 1032)[i], max_rank=rank,
                                        n_adapted=48, skip_seqs=3, name=f"set_k{k}")
             for i, k in enumerate(k_ins)]
    devs = [DeviceCase(c, DEV) for c in cases]

    def run_set():
        outs = [d.base0.clone() for d in devs]
        projs = [ml.make_projection(d.route, d.x, o, d.indices, d.row_adapter, c.top_k)
                 for c, d, o in zip(cases, devs, outs)]
        ml.mlora_gather_bgmv_set(projs)
        torch.cuda.synchronize()
        return [from_torch(o) for o in outs]

    res = run_set()
    for c, got in zip(cases, res):
        check(OracleView(c), got, c.base, f"{c.name} set, decode kernel")
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    stream = run_set()
    for c, a, b in zip(cases, res, stream):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), c.name


def test_set_graph_replay_reads_routing_on_device():
    """A projection set captured in a HIP graph (members through the decode
    kernel's body): every replay equals the eager call bit for bit, and a
    replay after the routing, the map and one table cell of a member are
    rewritten in place folds by the new contents."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase, from_torch, to_torch
    from tests.test_gpu_fold import check
    _need_gpu()
    cases = [workloads.make_gather_case(160 + i, n_seq=40, padded_n=44, top_k=8, n_route=64,
                                        k_in=(768, 2048)[i], n_out=(1032, 768)[i], max_rank=16,
                                        n_adapted=48, skip_seqs=3, name=f"graph_set_{i}")
             for i in range(2)]
    devs = [DeviceCase(c, DEV) for c in cases]
    pristine = [to_torch(c.base, "bf16", DEV) for c in cases]
    outs = [p.clone() for p in pristine]
    projs = [ml.make_projection(d.route, d.x, o, d.indices, d.row_adapter, c.top_k)
             for c, d, o in zip(cases, devs, outs)]
    ml.mlora_gather_bgmv_set(projs)
    torch.cuda.synchronize()
    eager = [from_torch(o) for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ml.mlora_gather_bgmv_set(projs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        for o, p in zip(outs, pristine):
            o.copy_(p)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(from_torch(o).view(np.uint16), e.view(np.uint16))
    # member 1: new routing, a new map and one live table cell cleared, in place
    c, d = cases[1], devs[1]
    rng = np.random.default_rng(161)
    new_idx = rng.integers(0, 64, size=c.indices.shape, dtype=np.int64).astype(np.int32)
    new_map = np.where(rng.random(d.row_adapter.numel()) < 0.3, -1, 1).astype(np.int32)
    d.indices.copy_(torch.from_numpy(new_idx))
    d.row_adapter.copy_(torch.from_numpy(new_map))
    live_e = int(np.flatnonzero(d.tables_host[0])[0])
    d.a_table[live_e] = 0
    for o, p in zip(outs, pristine):
        o.copy_(p)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(from_torch(outs[0]).view(np.uint16), eager[0].view(np.uint16))
    c2 = workloads.FoldCase(**{k: getattr(c, k) for k in c.__dataclass_fields__})
    c2.indices = new_idx
    view = OracleView(c2)
    view.row_adapter = new_map
    view.a_table = list(view.a_table)
    view.a_table[live_e] = 0
    check(view, from_torch(outs[1]), c.base, "set graph replay, new routing")
