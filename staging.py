"""Stage a seeded FoldCase on the GPU and run it through libmlora (used by the
GPU tests, the smoke check and the benchmark).

The tables and the per-row adapter map are built by the library's own host
functions (so the fold runs on exactly what the boundary produces); the
weights live in one pool tensor per matrix kind and the tables hold their
device addresses.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_expert_lora_amd as ml
from workloads import NULL_HANDLE, FoldCase


def to_torch(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Host array (bf16 bits as uint16, or float32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def from_torch(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array (bf16 as uint16 bits, float32 as float32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def u64_to_device(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint64).view(np.int64)).to(device)


class DeviceCase:
    """Everything one fold call needs, resident on the GPU."""

    def __init__(self, case: FoldCase, device="cuda", two_kernel: bool = True,
                 pipelined: bool = True):
        self.case = case
        self.device = device
        self.two_kernel = two_kernel
        self.pipelined = pipelined
        self._ws = None
        c = case
        self.tdtype = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        self.x = to_torch(c.x, c.dtype, device)
        self.a_pool = to_torch(c.a_pool, c.dtype, device)
        self.b_pool = to_torch(c.b_pool, c.dtype, device)
        self.base0 = to_torch(c.base, c.dtype, device)
        elt = 2 if c.dtype == "bf16" else 4
        a_stride = c.max_rank * c.k_in * elt
        b_stride = c.n_out * c.max_rank * elt

        def addr(pool, stride, h):
            return 0 if h == NULL_HANDLE else pool.data_ptr() + h * stride

        ids = np.array([e for (e, _, _, _) in c.entries], dtype=np.int32)
        a_addrs = np.array([addr(self.a_pool, a_stride, a) for (_, a, _, _) in c.entries],
                           dtype=np.uint64)
        b_addrs = np.array([addr(self.b_pool, b_stride, b) for (_, _, b, _) in c.entries],
                           dtype=np.uint64)
        scales = np.array([s for (_, _, _, s) in c.entries], dtype=np.float32)
        self.entries_host = (ids, a_addrs, b_addrs, scales)
        packed = ml.mlora_pack_expert_tables(ids, a_addrs, b_addrs, scales)
        if packed is None:
            at, bt, st, n = (np.zeros(0, np.uint64), np.zeros(0, np.uint64),
                             np.zeros(0, np.float32), 0)
        else:
            at, bt, st, n = packed
        self.tables_host = (at, bt, st, n)
        self.a_table = u64_to_device(np.concatenate([at, [0]]), device)
        self.b_table = u64_to_device(np.concatenate([bt, [0]]), device)
        self.scale_table = torch.from_numpy(np.concatenate([st, [0]]).astype(np.float32)).to(device)
        self.route = ml.make_route(self.a_table, self.b_table, self.scale_table, n, c.k_in,
                                   c.n_out, c.max_rank, self.tdtype)
        if c.map_kind == "decode":
            ra = ml.mlora_build_moe_row_adapter_decode(c.adapter_slots, c.padded_n, c.active,
                                                       c.has_moe_lora)
        else:
            ra = ml.mlora_build_moe_row_adapter_host(c.cu_seqlens, c.stream_slots)
            assert ra is not None
        self.row_adapter_host = ra
        # the map covers every x row (padding tokens of x beyond the map get -1)
        full = np.full(max(c.n_tokens, ra.shape[0]), -1, dtype=np.int32)
        full[: ra.shape[0]] = ra
        self.row_adapter = torch.from_numpy(full).to(device)
        if c.path == "gather":
            self.indices = torch.from_numpy(np.ascontiguousarray(c.indices, np.int32)).to(device)
        else:
            self.sorted_ids = torch.from_numpy(np.ascontiguousarray(c.sorted_ids, np.int32)).to(device)
            self.offsets = torch.from_numpy(np.ascontiguousarray(c.expert_offsets, np.int32)).to(device)
            self.windows = ml.mlora_grouped_down_windows(c.n_rows, c.cap)

    def workspace_for(self, windows=None) -> torch.Tensor:
        """A device workspace large enough for the call(s) (grown on demand):
        every window of a grouped case, or the gather call."""
        c = self.case
        if c.path == "gather":
            need = ml.mlora_gather_bgmv_workspace_bytes(c.indices.shape[0], c.k_in, c.max_rank)
        else:
            need = max([ml.mlora_grouped_down_workspace_bytes(s, e, c.max_rank)
                        for (s, e) in (windows or [])] +
                       [ml.mlora_grouped_down_all_workspace_bytes(c.n_rows, c.cap, c.max_rank)])
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def fold(self, base: torch.Tensor, windows=None, stream=None,
             two_kernel: bool = None, pipelined: bool = None) -> torch.Tensor:
        """Fold in place into ``base`` (a device tensor shaped like base_out).
        With ``two_kernel`` set the call gets a workspace (the two-kernel
        form where the library takes it), else none (one kernel); a grouped
        case with a workspace and no explicit windows folds every window in
        one pipelined call when ``pipelined`` is set, else window by window.
        None means the case's defaults."""
        c = self.case
        two = self.two_kernel if two_kernel is None else two_kernel
        if c.path == "gather":
            ws = self.workspace_for() if two else None
            ml.mlora_gather_bgmv(self.route, self.x, base, self.indices, self.row_adapter,
                                 c.top_k, workspace=ws, stream=stream)
        else:
            pipe = self.pipelined if pipelined is None else pipelined
            if two and pipe and windows is None:
                # every window in one pipelined call
                ml.mlora_grouped_down_all(self.route, self.x, base, self.offsets,
                                          self.sorted_ids, self.row_adapter, c.top_k, c.cap,
                                          self.workspace_for(self.windows), stream=stream)
                return base
            wins = self.windows if windows is None else windows
            ws = self.workspace_for(wins) if two else None
            for (s, e) in wins:
                ml.mlora_grouped_down(self.route, self.x, base, self.offsets, self.sorted_ids,
                                      self.row_adapter, c.top_k, s, e, workspace=ws,
                                      stream=stream)
        return base

    def run(self, base_host: np.ndarray = None, windows=None,
            two_kernel: bool = None, pipelined: bool = None) -> np.ndarray:
        base = self.base0.clone() if base_host is None else to_torch(base_host, self.case.dtype,
                                                                     self.device)
        self.fold(base, windows=windows, two_kernel=two_kernel, pipelined=pipelined)
        torch.cuda.synchronize()
        return from_torch(base)


class DeviceMultiCase:
    """A multi-adapter gather case (workloads.make_multi_gather_case) on the
    GPU: the weights in pools, the tables packed and the decode map built by
    the library's multi-adapter host functions."""

    def __init__(self, case: FoldCase, device="cuda"):
        self.case = case
        self.device = device
        c = case
        self.x = to_torch(c.x, c.dtype, device)
        self.a_pool = to_torch(c.a_pool, c.dtype, device)
        self.b_pool = to_torch(c.b_pool, c.dtype, device)
        self.base0 = to_torch(c.base, c.dtype, device)
        a_stride = c.max_rank * c.k_in * 2
        b_stride = c.n_out * c.max_rank * 2
        ent = c.notes["multi_entries"]
        slots = np.array([e[0] for e in ent], dtype=np.int32)
        ids = np.array([e[1] for e in ent], dtype=np.int32)
        a_addrs = np.array([self.a_pool.data_ptr() + e[2] * a_stride for e in ent], np.uint64)
        b_addrs = np.array([self.b_pool.data_ptr() + e[3] * b_stride for e in ent], np.uint64)
        scales = np.array([e[4] for e in ent], dtype=np.float32)
        at, bt, st, na, ne = ml.mlora_pack_expert_tables_multi(slots, ids, a_addrs, b_addrs,
                                                               scales)
        self.tables_host = (at, bt, st, na, ne)
        self.a_table = u64_to_device(np.concatenate([at, [0]]), device)
        self.b_table = u64_to_device(np.concatenate([bt, [0]]), device)
        self.scale_table = torch.from_numpy(np.concatenate([st, [0]]).astype(np.float32)).to(device)
        self.route = ml.make_multi_route(self.a_table, self.b_table, self.scale_table, na, ne,
                                         c.k_in, c.n_out, c.max_rank)
        self.row_adapter_host = ml.mlora_build_moe_row_adapter_decode_multi(
            c.adapter_slots, c.padded_n, c.notes["n_adapters"])
        self.row_adapter = torch.from_numpy(self.row_adapter_host).to(device)
        self.indices = torch.from_numpy(np.ascontiguousarray(c.indices, np.int32)).to(device)

    def run(self, base_host: np.ndarray = None) -> np.ndarray:
        base = self.base0.clone() if base_host is None else to_torch(base_host, self.case.dtype,
                                                                     self.device)
        ml.mlora_gather_bgmv_multi(self.route, self.x, base, self.indices, self.row_adapter,
                                   self.case.top_k)
        torch.cuda.synchronize()
        return from_torch(base)
