"""The grouped all-windows fold for callers that cannot allocate
(mlora_grouped_down_all_noalloc, the library's static device scratch) against
the entry point it varies (mlora_grouped_down_all with a caller workspace),
through the C ABI: the same bits, on two calls in a row, the second smaller
(its scratch then holds the first call's contents)."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.common import REL_L2_TOL, OracleView, parity_figures, to_f64

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _fold(dev, noalloc):
    import moe_expert_lora_amd as ml
    from staging import from_torch
    c = dev.case
    out = dev.base0.clone()
    if noalloc:
        ml.mlora_grouped_down_all_noalloc(dev.route, dev.x, out, dev.offsets, dev.sorted_ids,
                                          dev.row_adapter, c.top_k, c.cap)
    else:
        ml.mlora_grouped_down_all(dev.route, dev.x, out, dev.offsets, dev.sorted_ids,
                                  dev.row_adapter, c.top_k, c.cap, dev.workspace_for(dev.windows))
    torch.cuda.synchronize()
    return from_torch(out)


def _cases():
    big = workloads.prefill_grouped_down()   # two launch slots of 16384 rows, rank 32
    small = workloads.with_unnamed_rows(
        workloads.make_grouped_case(81, stream_lens=[700, 513], top_k=4, n_route=20, k_in=264,
                                    n_out=200, max_rank=48, routing="zipf", n_unadapted=3,
                                    cap=1000, name="noalloc_small"), 81, lead=9, tail=14,
        bad_frac=0.05)
    f32 = workloads.make_grouped_case(82, stream_lens=[40, 21], top_k=2, n_route=7, k_in=48,
                                      n_out=24, max_rank=8, dtype="f32", n_unadapted=1, cap=50,
                                      name="noalloc_f32")
    return [big, small, f32]


def test_noalloc_equals_workspace_entry_on_calls_in_a_row():
    from staging import DeviceCase
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for case in _cases():
        dev = DeviceCase(case, "cuda")
        want = _fold(dev, noalloc=False)
        got = _fold(dev, noalloc=True)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), case.name
        view = OracleView(case)
        ref = view.fold()
        rel, mx, ex = parity_figures(view, to_f64(got, case.dtype), ref, f"{case.name} noalloc")
        print(f"{case.name} noalloc: rel_l2={rel:.3e} max_abs={mx:.3e} max_abs/limit={ex:.3f}",
              flush=True)
        assert rel <= REL_L2_TOL and ex <= 1.0
        live = view.live_rows()
        assert np.array_equal(got[~live].view(np.uint8), case.base[~live].view(np.uint8))


def test_noalloc_rejects_more_than_its_scratch():
    """A call whose launch slots would not fit the scratch returns
    MLORA_ERR_CAPACITY and writes nothing."""
    import moe_expert_lora_amd as ml
    from staging import DeviceCase
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    case = workloads.make_grouped_case(83, stream_lens=[9000], top_k=8, n_route=16, k_in=8,
                                       n_out=8, max_rank=128, cap=72000, name="noalloc_too_big")
    assert ml.mlora_grouped_down_all_workspace_bytes(case.n_rows, case.cap, 128) > \
        ml.NOALLOC_SCRATCH_BYTES
    dev = DeviceCase(case, "cuda")
    out = dev.base0.clone()
    with pytest.raises(ml.MloraError) as ei:
        ml.mlora_grouped_down_all_noalloc(dev.route, dev.x, out, dev.offsets, dev.sorted_ids,
                                          dev.row_adapter, case.top_k, case.cap)
    assert ei.value.code == ml.MLORA_ERR_CAPACITY and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.equal(out, dev.base0)
