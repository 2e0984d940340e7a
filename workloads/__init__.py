"""Seeded synthetic inputs for the MoE expert-LoRA fold.

This module is shared by the oracle side and the device side, so it holds none
of the fold's arithmetic. It only:

* draws random numbers (NumPy PCG64, ``default_rng(seed)``),
* encodes drawn fp32 values as bf16 bit patterns (round to nearest even),
* lays the drawn routing out the way an MoE router hands it over: a top-k
  expert choice per token, and for prefill the stable sort of the flat
  ``(token, slot)`` rows by expert (``sorted_ids`` plus ``expert_offsets``).

The per-row adapter maps and the packed expert tables are *not* built here:
the generator returns their raw inputs (adapter slots, ``cu_seqlens``, the
packing entries) so that the code under test builds them.

Weights live in pools: ``a_pool[h]`` is ``A`` of handle ``h`` with shape
``[max_rank, k_in]`` and ``b_pool[h]`` is ``B`` with shape ``[n_out, max_rank]``.
A packing entry ``(expert_id, a_handle, b_handle, scale)`` names handles; handle
``-1`` stands for a null address (an unadapted cell).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

NULL_HANDLE = -1

Entry = Tuple[int, int, int, float]


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class FoldCase:
    """One seeded fold problem.

    ``path`` is ``"gather"`` (decode rows in flat ``(token, slot)`` order, the
    expert comes from ``indices``) or ``"grouped"`` (rows sorted by expert, the
    expert comes from the ``expert_offsets`` span).
    """

    name: str
    path: str
    dtype: str  # "f32" or "bf16": x, A, B and base_out share it
    seed: int
    top_k: int
    k_in: int
    n_out: int
    max_rank: int
    n_tokens: int
    x: np.ndarray  # [n_tokens, k_in]  float32 or uint16 bf16 bits
    a_pool: np.ndarray  # [n_handles, max_rank, k_in]
    b_pool: np.ndarray  # [n_handles, n_out, max_rank]
    entries: List[Entry]
    base: np.ndarray  # [n_rows, n_out]
    # per-row adapter map inputs
    map_kind: str  # "decode" or "host"
    adapter_slots: Optional[np.ndarray] = None  # decode: one per sequence
    padded_n: int = 0
    active: int = 1
    has_moe_lora: bool = True
    cu_seqlens: Optional[np.ndarray] = None  # host: [batch + 1]
    stream_slots: Optional[np.ndarray] = None  # host: [batch]
    # gather routing
    indices: Optional[np.ndarray] = None  # [n_slots] int32
    # grouped routing
    sorted_ids: Optional[np.ndarray] = None  # [n_rows] int32, flat (token, slot) id
    expert_offsets: Optional[np.ndarray] = None  # [n_route + 1] int32
    cap: int = 0  # window cap for grouped_down_windows
    notes: dict = field(default_factory=dict)

    @property
    def n_rows(self) -> int:
        return int(self.base.shape[0])

    @property
    def n_route(self) -> int:
        return 0 if self.expert_offsets is None else int(self.expert_offsets.shape[0] - 1)

    def with_base(self, base: np.ndarray) -> "FoldCase":
        c = FoldCase(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        c.base = base
        return c


# ----------------------------------------------------------------------------
# random draws
# ----------------------------------------------------------------------------

def topk_uniform(rng: np.random.Generator, n_tok: int, n_exp: int, k: int) -> np.ndarray:
    """Per token, ``k`` distinct experts drawn uniformly (no replacement)."""
    if n_tok == 0:
        return np.zeros((0, k), dtype=np.int32)
    keys = rng.random((n_tok, n_exp))
    return np.argsort(keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def topk_weighted(rng: np.random.Generator, n_tok: int, weights: np.ndarray, k: int) -> np.ndarray:
    """Per token, ``k`` distinct experts drawn without replacement with
    probabilities proportional to ``weights`` (Gumbel-top-k)."""
    u = rng.random((n_tok, weights.shape[0]))
    g = -np.log(-np.log(np.clip(u, 1e-300, 1.0 - 1e-16)))
    keys = np.log(weights)[None, :] + g
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def sorted_layout(indices_flat: np.ndarray, n_route: int) -> Tuple[np.ndarray, np.ndarray]:
    """Router output for prefill: flat row ids stably sorted by expert, and the
    ``[n_route + 1]`` span starts. Ids outside ``[0, n_route)`` are not expected."""
    order = np.argsort(indices_flat, kind="stable").astype(np.int32)
    counts = np.bincount(indices_flat, minlength=n_route)[:n_route]
    offsets = np.zeros(n_route + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return order, offsets.astype(np.int32)


def _values(rng, shape, std, dtype):
    v = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v = (v * np.float32(std)).astype(np.float32)
    return bf16_from_f32(v) if dtype == "bf16" else v


def _weights(rng, n_handles, r, k_in, n_out, dtype):
    a = _values(rng, (n_handles, r, k_in), 1.0 / np.sqrt(k_in), dtype)
    b = _values(rng, (n_handles, n_out, r), 0.05, dtype)
    return a, b


def _entries_for(rng, adapted: np.ndarray, scale_lo: float, scale_hi: float,
                 dup_frac: float = 0.0, zero_ids=()) -> Tuple[List[Entry], int]:
    """Packing entries for ``adapted`` ids (handle = position), optionally with
    decoy entries listed before the real one for a ``dup_frac`` share of ids,
    plus null entries for ``zero_ids``. Returns (entries, n_handles)."""
    n = len(adapted)
    scales = rng.uniform(scale_lo, scale_hi, size=n).astype(np.float32)
    n_dup = int(round(dup_frac * n))
    dup_pos = set(rng.choice(n, size=n_dup, replace=False).tolist()) if n_dup else set()
    decoy_scales = rng.uniform(scale_lo, scale_hi, size=max(n_dup, 1)).astype(np.float32)
    entries: List[Entry] = []
    next_handle = n
    d = 0
    for pos, e in enumerate(adapted.tolist()):
        if pos in dup_pos:
            entries.append((int(e), next_handle, next_handle, float(decoy_scales[d])))
            next_handle += 1
            d += 1
        entries.append((int(e), pos, pos, float(scales[pos])))
    for z in zero_ids:
        entries.append((int(z), NULL_HANDLE, NULL_HANDLE, 0.0))
    return entries, next_handle


# ----------------------------------------------------------------------------
# generic builders
# ----------------------------------------------------------------------------

def make_gather_case(seed: int, *, n_seq: int, padded_n: int, top_k: int, n_route: int,
                     k_in: int, n_out: int, max_rank: int, dtype: str = "bf16",
                     adapted: Optional[np.ndarray] = None, n_adapted: Optional[int] = None,
                     skip_seqs: int = 0, refuse_seqs: int = 0, scale=(0.5, 2.0),
                     zero_ids=(), dup_frac: float = 0.0, index_mode: str = "uniform",
                     active: int = 1, has_moe_lora: bool = True,
                     wild_index_frac: float = 0.0, n_slots: Optional[int] = None,
                     name: str = "gather") -> FoldCase:
    """Decode-shaped gather problem.

    Draw order: routing, slots, adapted set, scales, x, A, B, base.
    ``n_slots`` defaults to ``padded_n * top_k``; padding tokens get valid
    routing so that only the map skips them. ``wild_index_frac`` replaces a
    share of the indices by ids outside the table (negative or too large).
    """
    rng = np.random.default_rng(seed)
    if n_slots is None:
        n_slots = padded_n * top_k
    n_tok_x = max(padded_n, -(-n_slots // top_k)) if n_slots else padded_n
    if index_mode == "uniform":
        idx = topk_uniform(rng, n_tok_x, n_route, top_k).reshape(-1)[:n_slots]
    elif index_mode == "zero":
        idx = np.zeros(n_slots, dtype=np.int32)
        rng.random(1)
    else:
        raise ValueError(index_mode)
    idx = idx.astype(np.int32)
    if wild_index_frac > 0 and n_slots:
        m = rng.random(n_slots) < wild_index_frac
        wild = rng.choice(np.array([-1, -7, n_route, n_route + 5, 2**30], dtype=np.int64),
                          size=n_slots).astype(np.int32)
        idx = np.where(m, wild, idx).astype(np.int32)
    # adapter slots per sequence: active, Skip (-1) or Refuse (another slot)
    slots = np.full(n_seq, active, dtype=np.int32)
    pick = rng.permutation(n_seq)
    slots[pick[:skip_seqs]] = -1
    slots[pick[skip_seqs:skip_seqs + refuse_seqs]] = active + 1
    if adapted is None:
        na = n_route if n_adapted is None else n_adapted
        adapted = np.sort(rng.choice(n_route, size=na, replace=False)).astype(np.int32)
    entries, n_handles = _entries_for(rng, np.asarray(adapted), scale[0], scale[1],
                                      dup_frac=dup_frac, zero_ids=zero_ids)
    x = _values(rng, (n_tok_x, k_in), 1.0, dtype)
    a_pool, b_pool = _weights(rng, max(n_handles, 1), max_rank, k_in, n_out, dtype)
    base = _values(rng, (n_slots, n_out), 1.0, dtype)
    return FoldCase(name=name, path="gather", dtype=dtype, seed=seed, top_k=top_k,
                    k_in=k_in, n_out=n_out, max_rank=max_rank, n_tokens=n_tok_x, x=x,
                    a_pool=a_pool, b_pool=b_pool, entries=entries, base=base,
                    map_kind="decode", adapter_slots=slots, padded_n=padded_n,
                    active=active, has_moe_lora=has_moe_lora, indices=idx)


def make_grouped_case(seed: int, *, stream_lens, top_k: int, n_route: int, k_in: int,
                      n_out: int, max_rank: int, dtype: str = "bf16",
                      routing: str = "uniform", zipf_alpha: float = 1.1,
                      adapted: Optional[np.ndarray] = None, n_unadapted: int = 0,
                      force_unadapted=(), dup_frac: float = 0.0, scale=(0.5, 2.0),
                      stream_slot_values=None, cap: int = 8192, active: int = 1,
                      name: str = "grouped") -> FoldCase:
    """Prefill-shaped grouped problem over packed streams.

    Draw order: routing, streams (given), adapted set, scales, x, A, B, base.
    """
    rng = np.random.default_rng(seed)
    stream_lens = np.asarray(stream_lens, dtype=np.int64)
    n_tok = int(stream_lens.sum())
    if routing == "uniform":
        idx = topk_uniform(rng, n_tok, n_route, top_k)
    elif routing == "zipf":
        w = (np.arange(n_route, dtype=np.float64) + 1.0) ** (-zipf_alpha)
        idx = topk_weighted(rng, n_tok, w, top_k)
    else:
        raise ValueError(routing)
    flat = idx.reshape(-1).astype(np.int32)
    sorted_ids, offsets = sorted_layout(flat, n_route)
    cu = np.zeros(len(stream_lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(stream_lens)
    if stream_slot_values is None:
        stream_slots = np.full(len(stream_lens), active, dtype=np.int32)
    else:
        stream_slots = np.asarray(stream_slot_values, dtype=np.int32)
    if adapted is None:
        un = set(int(v) for v in force_unadapted)
        rest = [e for e in range(n_route) if e not in un]
        extra = n_unadapted - len(un)
        if extra > 0:
            un |= set(rng.choice(rest, size=extra, replace=False).tolist())
        adapted = np.array([e for e in range(n_route) if e not in un], dtype=np.int32)
    entries, n_handles = _entries_for(rng, np.asarray(adapted), scale[0], scale[1],
                                      dup_frac=dup_frac)
    x = _values(rng, (n_tok, k_in), 1.0, dtype)
    a_pool, b_pool = _weights(rng, max(n_handles, 1), max_rank, k_in, n_out, dtype)
    base = _values(rng, (n_tok * top_k, n_out), 1.0, dtype)
    c = FoldCase(name=name, path="grouped", dtype=dtype, seed=seed, top_k=top_k,
                 k_in=k_in, n_out=n_out, max_rank=max_rank, n_tokens=n_tok, x=x,
                 a_pool=a_pool, b_pool=b_pool, entries=entries, base=base,
                 map_kind="host", cu_seqlens=cu, stream_slots=stream_slots,
                 sorted_ids=sorted_ids, expert_offsets=offsets, cap=cap, active=active)
    c.notes["indices_flat"] = flat
    return c


def with_unnamed_rows(case: FoldCase, seed: int, lead: int, tail: int,
                      bad_frac: float) -> FoldCase:
    """A grouped case whose sorted rows also hold rows that name no token, as a
    router's padded sorted output does: ``lead`` rows before the first span and
    ``tail`` rows after the last one (ids drawn from -1, a valid id, or an id
    past the last token), and a ``bad_frac`` share of the rows inside the
    spans whose id is replaced by -1 or by an id at/after
    ``n_tokens * top_k``. Offsets shift by ``lead``; base_out grows to match
    (fresh draws for the new rows). Only routing and base rows change."""
    assert case.path == "grouped"
    rng = np.random.default_rng([seed, 7])
    n_flat = case.n_tokens * case.top_k
    ids = case.sorted_ids.astype(np.int64).copy()
    bad = rng.random(ids.shape[0]) < bad_frac
    wild = rng.choice(np.array([-1, n_flat, n_flat + case.top_k, n_flat + 12345]),
                      size=ids.shape[0])
    ids = np.where(bad, wild, ids)
    pool = np.array([-1, 0, n_flat - 1, n_flat, 2 ** 30])
    lead_ids = rng.choice(pool, size=lead)
    tail_ids = rng.choice(pool, size=tail)
    new_ids = np.concatenate([lead_ids, ids, tail_ids]).astype(np.int32)
    offsets = (case.expert_offsets.astype(np.int64) + lead).astype(np.int32)
    extra_lead = _values(rng, (lead, case.n_out), 1.0, case.dtype)
    extra_tail = _values(rng, (tail, case.n_out), 1.0, case.dtype)
    base = np.concatenate([extra_lead, case.base, extra_tail], axis=0)
    c = case.with_base(base)
    c.sorted_ids = new_ids
    c.expert_offsets = offsets
    c.name = case.name + "_unnamed"
    return c


# ----------------------------------------------------------------------------
# the workloads measured and checked at full size
# ----------------------------------------------------------------------------

def tiny_gather_f32() -> FoldCase:
    """Tiny fp32 gather: 4 tokens, top-2 of 4 experts, expert 3 packed with null
    cells, k_in=64, n_out=32, rank 8, sequence 1 is a Skip request."""
    rng_seed = 1
    c = make_gather_case(rng_seed, n_seq=4, padded_n=4, top_k=2, n_route=4, k_in=64,
                         n_out=32, max_rank=8, dtype="f32", adapted=np.array([0, 1, 2]),
                         zero_ids=(3,), name="tiny_gather_f32")
    # the recipe fixes the slots: [active, Skip, active, active]
    c.adapter_slots = np.array([1, -1, 1, 1], dtype=np.int32)
    return c


def decode_down_gather() -> FoldCase:
    """Qwen3-MoE-like decode down-proj gather: 64 sequences x top-8 over 128
    experts, padded to 80 tokens (640 rows), 96 adapted experts, 6 Skip
    sequences, k_in=768, n_out=2048, rank 16, bf16."""
    return make_gather_case(2, n_seq=64, padded_n=80, top_k=8, n_route=128, k_in=768,
                            n_out=2048, max_rank=16, n_adapted=96, skip_seqs=6,
                            name="decode_down_gather")


def prefill_stream_lens(seed: int = 3) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    while True:
        lens = rng.integers(256, 769, size=7)
        last = 4096 - int(lens.sum())
        if 256 <= last <= 768:
            return np.concatenate([lens, [last]]).astype(np.int64)


def prefill_grouped_down() -> FoldCase:
    """Prefill grouped down fold: 4096 tokens from 8 packed streams, top-8 of 128
    experts with Zipf(1.1) weights (32768 sorted rows), all adapted, k_in=768,
    n_out=2048, rank 32, bf16, window cap 8192."""
    return make_grouped_case(3, stream_lens=prefill_stream_lens(), top_k=8, n_route=128,
                             k_in=768, n_out=2048, max_rank=32, routing="zipf",
                             zipf_alpha=1.1, cap=8192, name="prefill_grouped_down")


def gateup_gather() -> FoldCase:
    """Gate/up gather (hidden -> intermediate): 256 sequences x top-8 (2048 rows),
    128 experts all adapted, k_in=2048, n_out=768, rank 64, scale U[0.25, 4]."""
    return make_gather_case(4, n_seq=256, padded_n=256, top_k=8, n_route=128, k_in=2048,
                            n_out=768, max_rank=64, scale=(0.25, 4.0),
                            name="gateup_gather")


def router_gather() -> FoldCase:
    """Router fold as a one-entry route: expert 0 over 8192 token rows, top_k=1,
    k_in=2048, n_out=128, rank 16. The map comes from one prefill stream."""
    c = make_gather_case(51, n_seq=1, padded_n=8192, top_k=1, n_route=1, k_in=2048,
                         n_out=128, max_rank=16, adapted=np.array([0]), index_mode="zero",
                         name="router_gather")
    c.map_kind = "host"
    c.cu_seqlens = np.array([0, 8192], dtype=np.int32)
    c.stream_slots = np.array([1], dtype=np.int32)
    c.adapter_slots = None
    return c


def mixed_grouped() -> FoldCase:
    """Mixed prefill grouped fold: 2048 tokens x top-8 (16384 sorted rows) over
    256 experts, 77 unadapted (id 255 among them), about 10% of adapted ids
    packed twice (a decoy first, the real pair last), k_in=1536, n_out=4096,
    rank 16, 8 streams of 256 tokens."""
    return make_grouped_case(52, stream_lens=[256] * 8, top_k=8, n_route=256, k_in=1536,
                             n_out=4096, max_rank=16, routing="uniform", n_unadapted=77,
                             force_unadapted=(255,), dup_frac=0.10, cap=8192,
                             name="mixed_grouped")


def make_multi_gather_case(seed: int, *, n_seq: int, padded_n: int, top_k: int, n_route: int,
                           k_in: int, n_out: int, max_rank: int, n_adapters: int,
                           adapted_frac: float = 0.75, skip_seqs: int = 0,
                           uninstalled_seqs: int = 0, dup_frac: float = 0.0,
                           scale=(0.5, 2.0), dtype: str = "bf16",
                           name: str = "multi_gather") -> FoldCase:
    """Decode-shaped gather problem over several installed adapters.

    Each adapter slot adapts its own seeded subset (adapted_frac) of the
    n_route experts with its own weights; the packing entries are
    (slot, expert, a_handle, b_handle, scale) in notes["multi_entries"]
    (a dup_frac share listed twice, a decoy first). Each sequence asks for a
    slot drawn uniformly from the installed ones; skip_seqs ask for none (-1)
    and uninstalled_seqs for the slot past the installed ones.
    Draw order: routing, slots, adapted sets, scales, x, A, B, base."""
    rng = np.random.default_rng(seed)
    n_slots = padded_n * top_k
    idx = topk_uniform(rng, padded_n, n_route, top_k).reshape(-1).astype(np.int32)
    slots = rng.integers(0, n_adapters, size=n_seq).astype(np.int32)
    pick = rng.permutation(n_seq)
    slots[pick[:skip_seqs]] = -1
    slots[pick[skip_seqs:skip_seqs + uninstalled_seqs]] = n_adapters
    entries: List[Tuple[int, int, int, int, float]] = []
    n_handles = 0
    for s_ in range(n_adapters):
        na = max(1, int(round(adapted_frac * n_route)))
        adapted = np.sort(rng.choice(n_route, size=na, replace=False))
        scales = rng.uniform(scale[0], scale[1], size=na).astype(np.float32)
        dups = rng.random(na) < dup_frac
        for j, e in enumerate(adapted.tolist()):
            if dups[j]:
                entries.append((s_, int(e), n_handles, n_handles,
                                float(rng.uniform(scale[0], scale[1]))))
                n_handles += 1
            entries.append((s_, int(e), n_handles, n_handles, float(scales[j])))
            n_handles += 1
    x = _values(rng, (padded_n, k_in), 1.0, dtype)
    a_pool, b_pool = _weights(rng, max(n_handles, 1), max_rank, k_in, n_out, dtype)
    base = _values(rng, (n_slots, n_out), 1.0, dtype)
    c = FoldCase(name=name, path="gather", dtype=dtype, seed=seed, top_k=top_k, k_in=k_in,
                 n_out=n_out, max_rank=max_rank, n_tokens=padded_n, x=x, a_pool=a_pool,
                 b_pool=b_pool, entries=[], base=base, map_kind="decode_multi",
                 adapter_slots=slots, padded_n=padded_n, indices=idx)
    c.notes["multi_entries"] = entries
    c.notes["n_adapters"] = n_adapters
    return c


def _with_routing_of(case: FoldCase, like: FoldCase) -> FoldCase:
    """`case` with the routing (expert ids, adapter slots) of `like`."""
    case.indices = like.indices.copy()
    case.adapter_slots = like.adapter_slots.copy()
    case.padded_n = like.padded_n
    return case


def decode_layer_cases(seed: int = 60, n_seq: int = 64, padded_n: int = 80, top_k: int = 8,
                       n_route: int = 128, n_adapted: int = 96, skip_seqs: int = 6,
                       hidden: int = 2048, inter: int = 768, rank: int = 16):
    """The four folds of one Qwen3-MoE-like decode layer over one batch, as
    gather problems: the router's one-entry route over the token rows
    (top_k 1, n_out = n_route expert logits), gate and up over the flat
    (token, slot) rows (hidden -> inter, one routing, their own adapted sets
    and weights), and down reading slot-major x (one inter-wide row per flat
    row, notes["x_rows"] = "row") back to hidden, on the same routing.
    Draws: gate's case, then up's, down's, down's slot-major x, the router's."""
    gate = make_gather_case(seed, n_seq=n_seq, padded_n=padded_n, top_k=top_k, n_route=n_route,
                            k_in=hidden, n_out=inter, max_rank=rank, n_adapted=n_adapted,
                            skip_seqs=skip_seqs, name="gate")
    up = _with_routing_of(make_gather_case(
        seed + 1, n_seq=n_seq, padded_n=padded_n, top_k=top_k, n_route=n_route, k_in=hidden,
        n_out=inter, max_rank=rank, n_adapted=n_adapted, skip_seqs=skip_seqs, name="up"), gate)
    down = _with_routing_of(make_gather_case(
        seed + 2, n_seq=n_seq, padded_n=padded_n, top_k=top_k, n_route=n_route, k_in=inter,
        n_out=hidden, max_rank=rank, n_adapted=n_adapted, skip_seqs=skip_seqs, name="down"),
        gate)
    rng = np.random.default_rng([seed, 3])
    down.x = _values(rng, (down.n_rows, inter), 1.0, "bf16")
    down.n_tokens = down.n_rows
    down.notes["x_rows"] = "row"
    router = make_gather_case(seed + 4, n_seq=n_seq, padded_n=padded_n, top_k=1, n_route=1,
                              k_in=hidden, n_out=n_route, max_rank=rank, adapted=np.array([0]),
                              index_mode="zero", name="router")
    # the router's token rows skip as the batch's sequences do (Skip, padding)
    router.adapter_slots = gate.adapter_slots.copy()
    return router, gate, up, down


def decode_multi_gather() -> FoldCase:
    """The decode down-proj gather batch (64 sequences x top-8 over 128
    experts, padded to 80 tokens, k_in 768, n_out 2048, rank 16) with four
    installed adapters, each adapting 75% of the experts with its own
    weights; 6 sequences ask for no adapter and 5 for one not installed."""
    return make_multi_gather_case(61, n_seq=64, padded_n=80, top_k=8, n_route=128, k_in=768,
                                  n_out=2048, max_rank=16, n_adapters=4, adapted_frac=0.75,
                                  skip_seqs=6, uninstalled_seqs=5, dup_frac=0.1,
                                  name="decode_multi_gather")


WORKLOADS = {
    "tiny_gather_f32": tiny_gather_f32,
    "decode_down_gather": decode_down_gather,
    "prefill_grouped_down": prefill_grouped_down,
    "gateup_gather": gateup_gather,
    "router_gather": router_gather,
    "mixed_grouped": mixed_grouped,
}
