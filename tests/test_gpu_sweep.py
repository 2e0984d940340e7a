"""GPU parity over a seeded sweep of shapes, through every launch form.

Each case draws its sizes from its seed (k_in and n_out multiples of 8 from
8 up to about 2000, or 8000 for the later seeds; ranks 1 to 128; top_k 1 to
8; routes of 1 to 40 experts, one-entry routes included; skipped, refused
and wild-index rows; slot counts that are not a multiple of top_k; grouped
windows from a few rows up) and is folded by
the default form and by every form the overrides can force (the grouped
expand's two unit orders must give the same bits); multi-adapter
cases add adapter counts, uninstalled slots and partly adapted slots. Every
result must meet the oracle bound, and every row that folds nothing must keep
its bits.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests.common import OracleView
from tests.test_gpu_fold import DEV, _need_gpu, check

pytestmark = pytest.mark.gpu


def _extra_seeds(name):
    """Seeds beyond the default lists, from an environment variable holding
    `first-last` (inclusive) or one seed, for a wider run by hand."""
    import os
    v = os.environ.get(name, "").strip()
    if not v:
        return []
    lo, _, hi = v.partition("-")
    return list(range(int(lo), int(hi or lo) + 1))


# seeds past the first 32 gather / 16 grouped ones draw k_in and n_out up to
# about 8000 (the hidden sizes of large MoE layers)
GATHER_SEEDS = list(range(44)) + _extra_seeds("MLORA_SWEEP_GATHER_SEEDS")
GROUPED_SEEDS = list(range(22)) + _extra_seeds("MLORA_SWEEP_GROUPED_SEEDS")

# forced gather forms: (label, overrides, run with a workspace)
GATHER_FORMS = [
    ("default", {}, True),
    ("no workspace", {}, False),
    ("streaming one kernel", {"MLORA_GATHER_RESIDENT": "0", "MLORA_GATHER_TWO": "0",
                              "MLORA_GATHER_DENSE": "0"}, True),
    ("two kernels", {"MLORA_GATHER_RESIDENT": "0", "MLORA_GATHER_TWO": "1",
                     "MLORA_GATHER_DENSE": "0"}, True),
    ("small chunks", {"MLORA_GATHER_SMALL": "1", "MLORA_GATHER_RESIDENT": "0",
                      "MLORA_GATHER_DENSE": "0"}, False),
]


def gather_case(seed):
    rng = np.random.default_rng([4242, seed])
    one_entry = seed % 6 == 5
    top_k = 1 if one_entry and seed % 12 == 5 else int(rng.integers(1, 9))
    n_route = 1 if one_entry else int(rng.integers(max(2, top_k), 41))
    n_seq = int(rng.integers(1, 65))
    padded_n = n_seq + int(rng.integers(0, 9))
    wide = seed >= 32
    k_in = 8 * int(rng.integers(1, 1001 if wide else 263))
    n_out = 8 * int(rng.integers(1, 1001 if wide else 138))
    max_rank = int(rng.choice([1, 3, 8, 12, 16, 17, 24, 32, 40, 56, 64, 72, 96, 100, 128]))
    kw = dict(n_seq=n_seq, padded_n=padded_n, top_k=top_k, n_route=n_route, k_in=k_in,
              n_out=n_out, max_rank=max_rank, skip_seqs=int(rng.integers(0, max(1, n_seq // 4))),
              name=f"sweep_gather_{seed}")
    if one_entry:
        kw.update(index_mode="zero", adapted=np.array([0]))
    else:
        kw.update(n_adapted=int(rng.integers(1, n_route + 1)),
                  refuse_seqs=int(rng.integers(0, 2)) if n_seq > 4 else 0,
                  wild_index_frac=float(rng.choice([0.0, 0.1])),
                  dup_frac=float(rng.choice([0.0, 0.2])))
        if seed % 4 == 3:  # slots not a multiple of top_k
            kw["n_slots"] = max(1, padded_n * top_k - int(rng.integers(1, top_k + 1)))
    return workloads.make_gather_case(7000 + seed, **kw)


def grouped_case(seed):
    rng = np.random.default_rng([4343, seed])
    n_streams = int(rng.integers(1, 5))
    lens = [int(v) for v in rng.integers(0, 160, size=n_streams)]
    if sum(lens) == 0:
        lens[0] = 1
    top_k = int(rng.integers(1, 9))
    n_route = int(rng.integers(top_k, top_k + 30))
    kw = dict(stream_lens=lens, top_k=top_k, n_route=n_route,
              k_in=8 * int(rng.integers(1, 1001 if seed >= 16 else 200)),
              n_out=8 * int(rng.integers(1, 1001 if seed >= 16 else 140)),
              max_rank=int(rng.choice([1, 5, 8, 16, 24, 32, 40, 48, 56, 64, 96, 128])),
              routing=str(rng.choice(["uniform", "zipf"])),
              n_unadapted=int(rng.integers(0, n_route // 2 + 1)),
              dup_frac=float(rng.choice([0.0, 0.2])),
              cap=int(rng.choice([3, 17, 64, 100, 1000])),
              stream_slot_values=[int(v) for v in rng.choice([1, 1, 1, -1], size=n_streams)],
              name=f"sweep_grouped_{seed}")
    return workloads.make_grouped_case(7100 + seed, **kw)


def _sentinel_run(view, dev, case, **kw):
    live = view.live_rows()
    if live.all():
        return
    base = case.base.copy()
    base.view(np.uint16)[~live] = 0x7F81
    got = dev.run(base, **kw)
    assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))


@pytest.mark.parametrize("seed", GATHER_SEEDS)
def test_gather_sweep_every_form(seed, overrides):
    _need_gpu()
    from staging import DeviceCase
    case = gather_case(seed)
    view = OracleView(case)
    dev = DeviceCase(case, DEV)
    for label, ov, ws in GATHER_FORMS:
        for k in ("MLORA_GATHER_RESIDENT", "MLORA_GATHER_TWO", "MLORA_GATHER_DENSE",
                  "MLORA_GATHER_SMALL"):
            if k in ov:
                overrides.set(k, ov[k])
            else:
                overrides.delete(k)
        check(view, dev.run(two_kernel=ws), case.base, f"{case.name} {label}")
    _sentinel_run(view, dev, case)


@pytest.mark.parametrize("seed", GROUPED_SEEDS)
def test_grouped_sweep_every_form(seed, overrides):
    _need_gpu()
    from staging import DeviceCase
    case = grouped_case(seed)
    view = OracleView(case)
    dev = DeviceCase(case, DEV)
    windows = view.windows()
    for label, kw in (("two kernels", dict(two_kernel=True, pipelined=False)),
                      ("one kernel", dict(two_kernel=False, pipelined=False)),
                      ("all windows", dict(two_kernel=True, pipelined=True))):
        check(view, dev.run(**kw), case.base, f"{case.name} {label}", windows=windows)
    # the expand units in block order and in contiguous XCD shares: the same bits
    forced = []
    for xcd in (0, 1):
        overrides.set("MLORA_EXPAND_XCD", xcd)
        forced.append(dev.run(two_kernel=True, pipelined=True))
    overrides.delete("MLORA_EXPAND_XCD")
    check(view, forced[0], case.base, f"{case.name} expand units in block order", windows=windows)
    assert np.array_equal(forced[0].view(np.uint16), forced[1].view(np.uint16))
    _sentinel_run(view, dev, case, two_kernel=True, pipelined=True)


MULTI_SEEDS = list(range(8)) + _extra_seeds("MLORA_SWEEP_MULTI_SEEDS")


def multi_case(seed):
    rng = np.random.default_rng([4444, seed])
    top_k = int(rng.integers(1, 9))
    n_seq = int(rng.integers(2, 49))
    return workloads.make_multi_gather_case(
        7200 + seed, n_seq=n_seq, padded_n=n_seq + int(rng.integers(0, 6)), top_k=top_k,
        n_route=int(rng.integers(top_k, 40)), k_in=8 * int(rng.integers(1, 257)),
        n_out=8 * int(rng.integers(1, 130)),
        max_rank=int(rng.choice([1, 7, 16, 24, 32, 64, 128])),
        n_adapters=int(rng.integers(1, 6)), adapted_frac=float(rng.choice([0.3, 0.75, 1.0])),
        skip_seqs=int(rng.integers(0, max(1, n_seq // 4))),
        uninstalled_seqs=int(rng.integers(0, 2)), dup_frac=float(rng.choice([0.0, 0.2])),
        name=f"sweep_multi_{seed}")


@pytest.mark.parametrize("seed", MULTI_SEEDS)
def test_multi_sweep(seed):
    """The multi-adapter fold over seeded shapes: the oracle bound and rows
    that fold nothing untouched."""
    _need_gpu()
    from oracle.case import OracleMultiView
    from staging import DeviceMultiCase
    from tests.test_gpu_multi import _check
    case = multi_case(seed)
    view, dev = OracleMultiView(case), DeviceMultiCase(case, DEV)
    _check(view, dev.run(), case.base, f"{case.name} R")
    live = view.live_rows()
    if not live.all():
        base = case.base.copy()
        base.view(np.uint16)[~live] = 0x7F81
        got = dev.run(base)
        assert np.array_equal(got[~live].view(np.uint8), base[~live].view(np.uint8))
