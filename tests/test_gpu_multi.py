"""GPU parity of the multi-adapter gather fold (mlora_gather_bgmv_multi)
against the fp64 multi-adapter oracle, through the C ABI: the oracle bound on
a random and a zero base, rows that fold nothing untouched bit for bit, the
same bits as one single-adapter call per slot on that slot's rows, and the
one-slot case equal to the single-adapter call."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.common import REL_L2_TOL, eval_margin, max_abs, max_abs_excess, rel_l2, to_f64
from tests.common import PARITY_LOG

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    ("decode_4ad", dict(n_seq=64, padded_n=80, top_k=8, n_route=128, k_in=768, n_out=2048,
                        max_rank=16, n_adapters=4, adapted_frac=0.75, skip_seqs=6,
                        uninstalled_seqs=5, dup_frac=0.1)),
    ("small_r32", dict(n_seq=30, padded_n=33, top_k=4, n_route=20, k_in=328, n_out=200,
                       max_rank=32, n_adapters=3, adapted_frac=0.6, skip_seqs=3,
                       uninstalled_seqs=2)),
    ("wide_r64", dict(n_seq=40, padded_n=40, top_k=2, n_route=12, k_in=2048, n_out=264,
                      max_rank=64, n_adapters=2, adapted_frac=0.9, skip_seqs=2)),
]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(view, got, base, label):
    ref = view.fold(base=base)
    g = to_f64(got, "bf16")
    eps = eval_margin(view.magnitude(), ref, view.case.k_in, view.case.max_rank)
    rel, mx = rel_l2(g, ref), max_abs(g, ref)
    ex = max_abs_excess(g, ref, "bf16", eps)
    PARITY_LOG.append((label, rel, mx, ex))
    print(f"{label}: rel_l2={rel:.3e} max_abs={mx:.3e} max_abs/limit={ex:.3f}", flush=True)
    assert rel <= REL_L2_TOL and ex <= 1.0, label
    live = view.live_rows()
    assert np.array_equal(got[~live].view(np.uint16), base[~live].view(np.uint16)), label


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_multi_parity(label, kw):
    from oracle.case import OracleMultiView
    from staging import DeviceMultiCase
    _need_gpu()
    c = workloads.make_multi_gather_case(210, name=label, **kw)
    view, dev = OracleMultiView(c), DeviceMultiCase(c, DEV)
    assert dev.row_adapter_host.tolist() == view.row_adapter.tolist()
    at, bt, st, na, ne = dev.tables_host
    assert (na, ne) == (view.n_adapters, view.n_experts)
    assert [int(v != 0) for v in at] == [int(v != 0) for v in view.a_table]
    _check(view, dev.run(), c.base, f"multi {label} R")
    zero = np.zeros_like(c.base)
    _check(view, dev.run(zero), zero, f"multi {label} Z")
    # rows that fold nothing keep a signalling-NaN sentinel
    live = view.live_rows()
    base = c.base.copy()
    base.view(np.uint16)[~live] = 0x7F81
    got = dev.run(base)
    assert np.array_equal(got[~live], base[~live])
    # every installed slot folds rows (the batch mixes adapters)
    used = {int(s) for s in dev.row_adapter_host if s >= 0}
    assert used == set(range(kw["n_adapters"]))


@pytest.mark.parametrize("label,kw", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_multi_equals_one_single_call_per_slot(label, kw):
    """The multi fold gives the bits of the single-adapter fold run once per
    slot, each over that slot's rows (the map of other slots set to -1), on
    that slot's tables: the rows a phase-1 engine would refuse fold with
    their own adapter."""
    import moe_expert_lora_amd as ml
    from staging import DeviceMultiCase, from_torch, u64_to_device
    _need_gpu()
    c = workloads.make_multi_gather_case(211, name=label, **kw)
    dev = DeviceMultiCase(c, DEV)
    got = dev.run()
    at, bt, st, na, ne = dev.tables_host
    out = dev.base0.clone()
    for s in range(na):
        cells = slice(s * ne, (s + 1) * ne)
        a_t = u64_to_device(np.concatenate([at[cells], [0]]), DEV)
        b_t = u64_to_device(np.concatenate([bt[cells], [0]]), DEV)
        s_t = torch.from_numpy(np.concatenate([st[cells], [0]]).astype(np.float32)).to(DEV)
        route = ml.make_route(a_t, b_t, s_t, ne, c.k_in, c.n_out, c.max_rank, torch.bfloat16)
        m = torch.from_numpy(np.where(dev.row_adapter_host == s, 0, -1).astype(np.int32)).to(DEV)
        ml.mlora_gather_bgmv(route, dev.x, out, dev.indices, m, c.top_k)
        torch.cuda.synchronize()
    assert np.array_equal(from_torch(out).view(np.uint16), got.view(np.uint16))


@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_multi_decode_kernel_equals_streaming_kernel(label, kw, overrides):
    """The multi-adapter cells run through the decode kernel (weights in
    registers) where they fit and through the streaming kernel when that one
    is forced (MLORA_GATHER_RESIDENT=0): the same bits, and the forced form
    meets the oracle bound on its own."""
    from oracle.case import OracleMultiView
    from staging import DeviceMultiCase
    _need_gpu()
    c = workloads.make_multi_gather_case(212, name=label, **kw)
    view, dev = OracleMultiView(c), DeviceMultiCase(c, DEV)
    default = dev.run()
    overrides.set("MLORA_GATHER_RESIDENT", "0")
    streaming = dev.run()
    _check(view, streaming, c.base, f"multi {label} streaming")
    assert np.array_equal(default.view(np.uint16), streaming.view(np.uint16))


@pytest.mark.parametrize("label,kw", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_multi_graph_replay_reads_routing_on_device(label, kw):
    """The multi-adapter fold captured in a HIP graph: every replay (with eager
    work and syncs between) equals the eager fold bit for bit, and a replay
    after the routing, the map and one table cell are rewritten in place folds
    by the new contents (the oracle bound on the new case)."""
    from oracle.case import OracleMultiView
    from staging import DeviceMultiCase, from_torch, to_torch
    _need_gpu()
    c = workloads.make_multi_gather_case(213, name=label, **kw)
    dev = DeviceMultiCase(c, DEV)
    eager = dev.run()
    import moe_expert_lora_amd as ml
    pristine = to_torch(c.base, "bf16", DEV)
    base = pristine.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            ml.mlora_gather_bgmv_multi(dev.route, dev.x, base, dev.indices, dev.row_adapter,
                                       c.top_k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        base.copy_(pristine)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_torch(base).view(np.uint16), eager.view(np.uint16))
    # new routing, a new map (Skip, every installed slot, one slot past them)
    # and one live cell cleared, all written in place
    na, ne = dev.tables_host[3], dev.tables_host[4]
    rng = np.random.default_rng(214)
    new_idx = rng.integers(0, ne, size=c.indices.shape, dtype=np.int64).astype(np.int32)
    new_map = rng.integers(-1, na + 1, size=dev.row_adapter.numel()).astype(np.int32)
    dev.indices.copy_(torch.from_numpy(new_idx))
    dev.row_adapter.copy_(torch.from_numpy(new_map))
    live_cell = int(np.flatnonzero(dev.tables_host[0])[0])
    dev.a_table[live_cell] = 0
    base.copy_(pristine)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    c2 = workloads.FoldCase(**{k: getattr(c, k) for k in c.__dataclass_fields__})
    c2.indices = new_idx
    view = OracleMultiView(c2)
    view.row_adapter = new_map
    view.a_table = list(view.a_table)
    view.a_table[live_cell] = 0
    _check(view, from_torch(base), c.base, f"multi {label} graph replay, new routing")
