"""Python binding of libmlora.so: the MoE expert-LoRA fold for MI355X (gfx950).

Argument marshalling only. Every function has the name of the C entry point it
calls (include/mlora.h); host functions take and return NumPy arrays, the two
device folds take PyTorch tensors (used only for device memory and the current
stream) and enqueue the library's HIP kernels. There is no fallback path: when
libmlora.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmlora.so")

MLORA_OK = 0
MLORA_NONE = 1
MLORA_ERR_INVALID = -1
MLORA_ERR_REFUSE = -2
MLORA_ERR_CAPACITY = -3
MLORA_ERR_HIP = -4

MLORA_ROUTE_FOLD = 0
MLORA_ROUTE_SKIP = 1
MLORA_ROUTE_REFUSE = 2

MLORA_F32 = 0
MLORA_BF16 = 1

# every symbol include/mlora.h declares
EXPORTS = (
    "mlora_resolve_moe_lora_route",
    "mlora_ensure_decode_route_servable",
    "mlora_pack_expert_tables",
    "mlora_build_moe_row_adapter_host",
    "mlora_build_moe_row_adapter_decode",
    "mlora_grouped_down_windows",
    "mlora_grouped_down_wc",
    "mlora_gather_row_token",
    "mlora_m_tile",
    "mlora_last_error",
    "mlora_gather_bgmv",
    "mlora_grouped_down",
    "mlora_grouped_down_workspace_bytes",
    "mlora_gather_bgmv_workspace_bytes",
    "mlora_grouped_down_all",
    "mlora_grouped_down_all_workspace_bytes",
    "mlora_reload_launch_overrides",
    "mlora_grouped_down_all_noalloc",
    "mlora_apply_expert_lora_sorted",
    "mlora_gather_bgmv_set",
    "mlora_resolve_moe_lora_route_multi",
    "mlora_build_moe_row_adapter_decode_multi",
    "mlora_pack_expert_tables_multi",
    "mlora_gather_bgmv_multi",
)


class MloraError(RuntimeError):
    """A libmlora call returned an error code."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class ExpertRoute(ctypes.Structure):
    """``mlora_expert_route``: device tables plus dims of one projection."""

    _fields_ = [
        ("a_table", ctypes.c_void_p),
        ("b_table", ctypes.c_void_p),
        ("scale_table", ctypes.c_void_p),
        ("n_experts", ctypes.c_int32),
        ("k_in", ctypes.c_int32),
        ("n_out", ctypes.c_int32),
        ("max_rank", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class MultiRoute(ctypes.Structure):
    """``mlora_multi_route``: device tables of n_adapters x n_experts cells."""

    _fields_ = [
        ("a_table", ctypes.c_void_p),
        ("b_table", ctypes.c_void_p),
        ("scale_table", ctypes.c_void_p),
        ("n_adapters", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("k_in", ctypes.c_int32),
        ("n_out", ctypes.c_int32),
        ("max_rank", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class Projection(ctypes.Structure):
    """``mlora_projection``: one gather call of a projection set."""

    _fields_ = [
        ("route", ctypes.POINTER(ExpertRoute)),
        ("x", ctypes.c_void_p),
        ("x_rows", ctypes.c_int64),
        ("x_ld", ctypes.c_int64),
        ("x_by_row", ctypes.c_int32),
        ("base_out", ctypes.c_void_p),
        ("out_ld", ctypes.c_int64),
        ("indices", ctypes.c_void_p),
        ("row_adapter", ctypes.c_void_p),
        ("map_len", ctypes.c_int64),
        ("n_slots", ctypes.c_int64),
        ("top_k", ctypes.c_int32),
    ]


_lib: Optional[ctypes.CDLL] = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_f32p = ctypes.POINTER(ctypes.c_float)


def load() -> ctypes.CDLL:
    """Load libmlora.so (once). Raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m moe_expert_lora_amd.build`")
    # PyTorch ships its own HIP runtime; load it first so that this library
    # binds to the same runtime instance that owns the tensors and streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
    sig = {
        "mlora_resolve_moe_lora_route": (i32, [i32, i32, i32]),
        "mlora_ensure_decode_route_servable": (i32, [i32]),
        "mlora_pack_expert_tables": (i32, [_i32p, _u64p, _u64p, _f32p, i64, _u64p, _u64p,
                                           _f32p, i64, _i32p]),
        "mlora_build_moe_row_adapter_host": (i32, [_i32p, i64, _i32p, i64, _i32p, i64, _i64p]),
        "mlora_build_moe_row_adapter_decode": (i32, [_i32p, i64, i64, i32, i32, _i32p]),
        "mlora_grouped_down_windows": (i32, [i64, i64, _i64p, _i64p, i64, _i64p]),
        "mlora_grouped_down_wc": (u32, [i64, i64]),
        "mlora_gather_row_token": (i32, [i32, i32]),
        "mlora_m_tile": (i32, []),
        "mlora_last_error": (ctypes.c_char_p, []),
        "mlora_gather_bgmv": (i32, [ctypes.POINTER(ExpertRoute), vp, i64, vp, vp, vp, i64,
                                    i32, vp, ctypes.c_uint64, vp]),
        "mlora_gather_bgmv_workspace_bytes": (ctypes.c_uint64, [i64, i32, i32]),
        "mlora_grouped_down": (i32, [ctypes.POINTER(ExpertRoute), vp, i64, vp, i64, vp, i32,
                                     vp, vp, i32, i64, i64, vp, ctypes.c_uint64, vp]),
        "mlora_grouped_down_workspace_bytes": (ctypes.c_uint64, [i64, i64, i32]),
        "mlora_grouped_down_all": (i32, [ctypes.POINTER(ExpertRoute), vp, i64, vp, i64, vp, i32,
                                         vp, vp, i32, i64, vp, ctypes.c_uint64, vp]),
        "mlora_grouped_down_all_workspace_bytes": (ctypes.c_uint64, [i64, i64, i32]),
        "mlora_reload_launch_overrides": (None, []),
        "mlora_grouped_down_all_noalloc": (i32, [ctypes.POINTER(ExpertRoute), vp, i64, vp, i64,
                                                 vp, i32, vp, vp, i32, i64, vp]),
        "mlora_gather_bgmv_set": (i32, [ctypes.POINTER(Projection), i32, vp]),
        "mlora_resolve_moe_lora_route_multi": (i32, [i32, i32]),
        "mlora_build_moe_row_adapter_decode_multi": (i32, [_i32p, i64, i64, i32, _i32p]),
        "mlora_pack_expert_tables_multi": (i32, [_i32p, _i32p, _u64p, _u64p, _f32p, i64, _u64p,
                                                 _u64p, _f32p, i64, _i32p, _i32p]),
        "mlora_gather_bgmv_multi": (i32, [ctypes.POINTER(MultiRoute), vp, i64, vp, vp, vp, i64,
                                          i32, vp]),
        "mlora_apply_expert_lora_sorted": (i32, [ctypes.POINTER(ExpertRoute), vp, i64, vp, i64,
                                                 vp, _i32p, i32, _u64p, _u64p, vp, vp, i32, vp,
                                                 ctypes.c_uint64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _err(code: int) -> MloraError:
    return MloraError(code, load().mlora_last_error().decode(errors="replace"))


def _arr(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=dtype))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype)) if a.size else None


# ---------------------------------------------------------------------------
# host functions
# ---------------------------------------------------------------------------

def mlora_resolve_moe_lora_route(adapter_slot: int, active: int, has_moe_lora: bool) -> int:
    return int(load().mlora_resolve_moe_lora_route(adapter_slot, active, int(bool(has_moe_lora))))


def mlora_ensure_decode_route_servable(route: int) -> None:
    rc = load().mlora_ensure_decode_route_servable(route)
    if rc != MLORA_OK:
        raise _err(rc)


def mlora_pack_expert_tables(expert_ids, a_addrs, b_addrs, scales):
    """Returns None for no entries, else (a_table, b_table, scale_table, n_experts)."""
    ids = _arr(expert_ids, np.int32)
    a = _arr(a_addrs, np.uint64)
    b = _arr(b_addrs, np.uint64)
    s = _arr(scales, np.float32)
    n_entries = ids.shape[0]
    if not (a.shape[0] == b.shape[0] == s.shape[0] == n_entries):
        raise ValueError("entry arrays differ in length")
    lib = load()
    n = ctypes.c_int32(0)
    rc = lib.mlora_pack_expert_tables(_ptr(ids, ctypes.c_int32), _ptr(a, ctypes.c_uint64),
                                      _ptr(b, ctypes.c_uint64), _ptr(s, ctypes.c_float),
                                      n_entries, None, None, None, 0, ctypes.byref(n))
    if rc == MLORA_NONE:
        return None
    if rc != MLORA_ERR_CAPACITY:
        raise _err(rc)
    at = np.zeros(n.value, dtype=np.uint64)
    bt = np.zeros(n.value, dtype=np.uint64)
    st = np.zeros(n.value, dtype=np.float32)
    rc = lib.mlora_pack_expert_tables(_ptr(ids, ctypes.c_int32), _ptr(a, ctypes.c_uint64),
                                      _ptr(b, ctypes.c_uint64), _ptr(s, ctypes.c_float),
                                      n_entries, _ptr(at, ctypes.c_uint64),
                                      _ptr(bt, ctypes.c_uint64), _ptr(st, ctypes.c_float),
                                      n.value, ctypes.byref(n))
    if rc != MLORA_OK:
        raise _err(rc)
    return at, bt, st, int(n.value)


def mlora_build_moe_row_adapter_host(cu_seqlens, adapter_slots) -> Optional[np.ndarray]:
    """Returns None when the builder rejects its input, else the int32 map."""
    cu = _arr(cu_seqlens, np.int32)
    sl = _arr(adapter_slots, np.int32)
    lib = load()
    total = ctypes.c_int64(0)
    rc = lib.mlora_build_moe_row_adapter_host(_ptr(cu, ctypes.c_int32), cu.shape[0],
                                              _ptr(sl, ctypes.c_int32), sl.shape[0], None, 0,
                                              ctypes.byref(total))
    if rc == MLORA_NONE:
        return None
    out = np.zeros(max(total.value, 0), dtype=np.int32)
    if rc == MLORA_ERR_CAPACITY:
        rc = lib.mlora_build_moe_row_adapter_host(_ptr(cu, ctypes.c_int32), cu.shape[0],
                                                  _ptr(sl, ctypes.c_int32), sl.shape[0],
                                                  _ptr(out, ctypes.c_int32), out.shape[0],
                                                  ctypes.byref(total))
    if rc != MLORA_OK:
        raise _err(rc)
    return out[: total.value]


def mlora_build_moe_row_adapter_decode(adapter_slots, padded_n: int, active: int,
                                       has_moe_lora: bool) -> np.ndarray:
    sl = _arr(adapter_slots, np.int32)
    out = np.zeros(int(padded_n), dtype=np.int32)
    rc = load().mlora_build_moe_row_adapter_decode(_ptr(sl, ctypes.c_int32), sl.shape[0],
                                                   int(padded_n), int(active),
                                                   int(bool(has_moe_lora)),
                                                   _ptr(out, ctypes.c_int32))
    if rc != MLORA_OK:
        raise _err(rc)
    return out


def mlora_grouped_down_windows(total_rows: int, cap: int) -> List[Tuple[int, int]]:
    lib = load()
    n = ctypes.c_int64(0)
    rc = lib.mlora_grouped_down_windows(int(total_rows), int(cap), None, None, 0,
                                        ctypes.byref(n))
    if rc == MLORA_OK:
        return []
    if rc != MLORA_ERR_CAPACITY:
        raise _err(rc)
    s = np.zeros(n.value, dtype=np.int64)
    e = np.zeros(n.value, dtype=np.int64)
    rc = lib.mlora_grouped_down_windows(int(total_rows), int(cap), _ptr(s, ctypes.c_int64),
                                        _ptr(e, ctypes.c_int64), n.value, ctypes.byref(n))
    if rc != MLORA_OK:
        raise _err(rc)
    return [(int(a), int(b)) for a, b in zip(s, e)]


def mlora_grouped_down_wc(row_offset: int, row_end: int) -> int:
    return int(load().mlora_grouped_down_wc(int(row_offset), int(row_end)))


def mlora_gather_row_token(row: int, top_k: int) -> int:
    return int(load().mlora_gather_row_token(int(row), int(top_k)))


def mlora_m_tile() -> int:
    return int(load().mlora_m_tile())


def mlora_reload_launch_overrides() -> None:
    """Re-read the MLORA_* launch-shape overrides from the environment."""
    load().mlora_reload_launch_overrides()


# ---------------------------------------------------------------------------
# device folds
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MLORA_BF16
    if t.dtype == torch.float32:
        return MLORA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_route(a_table, b_table, scale_table, n_experts: int, k_in: int, n_out: int,
               max_rank: int, dtype) -> ExpertRoute:
    """Route struct over device tables (uint64/int64, uint64/int64, float32
    tensors with n_experts entries). The caller keeps the tensors alive."""
    import torch
    for t in (a_table, b_table, scale_table):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("route tables must be contiguous device tensors")
    if scale_table.dtype != torch.float32:
        raise TypeError("scale_table must be float32")
    code = dtype if isinstance(dtype, int) else (
        MLORA_BF16 if dtype == torch.bfloat16 else MLORA_F32)
    return ExpertRoute(a_table.data_ptr(), b_table.data_ptr(), scale_table.data_ptr(),
                       int(n_experts), int(k_in), int(n_out), int(max_rank), code)


def _stream_handle(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dev(t, name, dtype=None):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    return t.data_ptr()


def mlora_gather_bgmv_workspace_bytes(n_slots: int, k_in: int, max_rank: int) -> int:
    """Workspace bytes the two-kernel gather fold may use."""
    return int(load().mlora_gather_bgmv_workspace_bytes(int(n_slots), int(k_in), int(max_rank)))


def mlora_gather_bgmv(route: ExpertRoute, x, base_out, indices, row_adapter, top_k: int,
                      workspace=None, stream=None) -> None:
    """Gather fold of every flat row of ``base_out`` [n_slots, n_out], in place.

    ``workspace``: None (one kernel) or a contiguous device tensor of at least
    ``mlora_gather_bgmv_workspace_bytes`` bytes (two kernels where that pays)."""
    import torch
    if _dtype_code(x) != route.dtype or _dtype_code(base_out) != route.dtype:
        raise TypeError("x / base_out dtype differs from the route's")
    if x.dim() != 2 or base_out.dim() != 2:
        raise ValueError("x and base_out must be 2-D")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    n_slots = base_out.shape[0]
    if indices.numel() != n_slots:
        raise ValueError("indices must have one entry per base_out row")
    if row_adapter.numel() < x.shape[0]:
        raise ValueError("row_adapter must cover every x row")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().mlora_gather_bgmv(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"),
        _dev(indices, "indices", torch.int32), _dev(row_adapter, "row_adapter", torch.int32),
        n_slots, int(top_k), ws_ptr, ws_bytes, _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


def mlora_grouped_down_workspace_bytes(row_offset: int, row_end: int, max_rank: int) -> int:
    """Workspace bytes of the two-kernel grouped fold on [row_offset, row_end)."""
    return int(load().mlora_grouped_down_workspace_bytes(int(row_offset), int(row_end),
                                                         int(max_rank)))


def mlora_grouped_down(route: ExpertRoute, x, base_out, expert_offsets, sorted_ids,
                       row_adapter, top_k: int, row_offset: int, row_end: int,
                       workspace=None, stream=None) -> None:
    """Grouped fold of sorted rows [row_offset, row_end) of ``base_out``, in place.

    ``workspace``: None (one kernel) or a contiguous device tensor of at least
    ``mlora_grouped_down_workspace_bytes`` bytes (two kernels)."""
    import torch
    if _dtype_code(x) != route.dtype or _dtype_code(base_out) != route.dtype:
        raise TypeError("x / base_out dtype differs from the route's")
    if x.dim() != 2 or base_out.dim() != 2:
        raise ValueError("x and base_out must be 2-D")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    n_rows = base_out.shape[0]
    if sorted_ids.numel() != n_rows:
        raise ValueError("sorted_ids must have one entry per base_out row")
    if row_adapter.numel() < x.shape[0]:
        raise ValueError("row_adapter must cover every x row")
    n_route = expert_offsets.numel() - 1
    if n_route < 0:
        raise ValueError("expert_offsets needs at least one entry")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().mlora_grouped_down(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"), n_rows,
        _dev(expert_offsets, "expert_offsets", torch.int32), int(n_route),
        _dev(sorted_ids, "sorted_ids", torch.int32),
        _dev(row_adapter, "row_adapter", torch.int32), int(top_k), int(row_offset),
        int(row_end), ws_ptr, ws_bytes, _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


def mlora_grouped_down_all_workspace_bytes(n_rows: int, cap: int, max_rank: int) -> int:
    """Workspace bytes of the pipelined all-windows grouped fold."""
    return int(load().mlora_grouped_down_all_workspace_bytes(int(n_rows), int(cap),
                                                             int(max_rank)))


def mlora_grouped_down_all(route: ExpertRoute, x, base_out, expert_offsets, sorted_ids,
                           row_adapter, top_k: int, cap: int, workspace, stream=None) -> None:
    """Grouped fold of every sorted row of ``base_out``, windows of ``cap`` rows
    pipelined; ``workspace`` a contiguous device tensor of at least
    ``mlora_grouped_down_all_workspace_bytes`` bytes (bf16 routes)."""
    import torch
    if _dtype_code(x) != route.dtype or _dtype_code(base_out) != route.dtype:
        raise TypeError("x / base_out dtype differs from the route's")
    if x.dim() != 2 or base_out.dim() != 2:
        raise ValueError("x and base_out must be 2-D")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    n_rows = base_out.shape[0]
    if sorted_ids.numel() != n_rows:
        raise ValueError("sorted_ids must have one entry per base_out row")
    if row_adapter.numel() < x.shape[0]:
        raise ValueError("row_adapter must cover every x row")
    n_route = expert_offsets.numel() - 1
    if n_route < 0:
        raise ValueError("expert_offsets needs at least one entry")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().mlora_grouped_down_all(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"), n_rows,
        _dev(expert_offsets, "expert_offsets", torch.int32), int(n_route),
        _dev(sorted_ids, "sorted_ids", torch.int32),
        _dev(row_adapter, "row_adapter", torch.int32), int(top_k), int(cap), ws_ptr, ws_bytes,
        _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


NOALLOC_SCRATCH_BYTES = 32 << 20  # MLORA_NOALLOC_SCRATCH_BYTES


def mlora_grouped_down_all_noalloc(route: ExpertRoute, x, base_out, expert_offsets, sorted_ids,
                                   row_adapter, top_k: int, cap: int, stream=None) -> None:
    """mlora_grouped_down_all without a workspace: the library's static device
    scratch holds the launch slots (for callers that cannot allocate)."""
    import torch
    if _dtype_code(x) != route.dtype or _dtype_code(base_out) != route.dtype:
        raise TypeError("x / base_out dtype differs from the route's")
    if x.dim() != 2 or base_out.dim() != 2:
        raise ValueError("x and base_out must be 2-D")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    n_rows = base_out.shape[0]
    if sorted_ids.numel() != n_rows:
        raise ValueError("sorted_ids must have one entry per base_out row")
    if row_adapter.numel() < x.shape[0]:
        raise ValueError("row_adapter must cover every x row")
    n_route = expert_offsets.numel() - 1
    if n_route < 0:
        raise ValueError("expert_offsets needs at least one entry")
    rc = load().mlora_grouped_down_all_noalloc(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"), n_rows,
        _dev(expert_offsets, "expert_offsets", torch.int32), int(n_route),
        _dev(sorted_ids, "sorted_ids", torch.int32),
        _dev(row_adapter, "row_adapter", torch.int32), int(top_k), int(cap),
        _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


def mlora_apply_expert_lora_sorted(route: ExpertRoute, x, base_out, expert_offsets,
                                   expert_offsets_host, a_table_host, b_table_host, sorted_ids,
                                   row_adapter, top_k: int, workspace=None, stream=None) -> None:
    """The host-loop sorted fold: one grouped launch per adapted expert's span,
    the spans and table cells given as host arrays (the caller copied the
    offsets to the host)."""
    import torch
    if _dtype_code(x) != route.dtype or _dtype_code(base_out) != route.dtype:
        raise TypeError("x / base_out dtype differs from the route's")
    n_rows = base_out.shape[0]
    if sorted_ids.numel() != n_rows:
        raise ValueError("sorted_ids must have one entry per base_out row")
    off_h = _arr(expert_offsets_host, np.int32)
    n_route = off_h.shape[0] - 1
    if n_route < 0 or expert_offsets.numel() != off_h.shape[0]:
        raise ValueError("host and device offsets differ in length")
    at = _arr(a_table_host, np.uint64)
    bt = _arr(b_table_host, np.uint64)
    if at.shape[0] < route.n_experts or bt.shape[0] < route.n_experts:
        raise ValueError("host tables shorter than n_experts")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = load().mlora_apply_expert_lora_sorted(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"), n_rows,
        _dev(expert_offsets, "expert_offsets", torch.int32), _ptr(off_h, ctypes.c_int32),
        int(n_route), _ptr(at, ctypes.c_uint64), _ptr(bt, ctypes.c_uint64),
        _dev(sorted_ids, "sorted_ids", torch.int32),
        _dev(row_adapter, "row_adapter", torch.int32), int(top_k), ws_ptr, ws_bytes,
        _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


def _rows_2d(t, name):
    """(data pointer, rows, row stride in elements) of a 2-D device tensor
    whose rows are contiguous (a column slice of a wider tensor is fine)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.shape[0] == 0:  # no rows: the strides say nothing
        return t.data_ptr(), 0, t.shape[1]
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")
    return t.data_ptr(), t.shape[0], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def make_projection(route: ExpertRoute, x, base_out, indices, row_adapter, top_k: int,
                    x_by_row: bool = False) -> Projection:
    """One projection of a set: `x` and `base_out` are 2-D bf16 device tensors
    with contiguous rows (their row strides become x_ld / out_ld), `indices`
    one int32 per base_out row, `row_adapter` the int32 per-token map. The
    caller keeps the tensors and the route alive while the set is used."""
    import torch
    if x.dtype != torch.bfloat16 or base_out.dtype != torch.bfloat16:
        raise TypeError("a projection set is bf16")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    xp, x_rows, x_ld = _rows_2d(x, "x")
    op, n_slots, out_ld = _rows_2d(base_out, "base_out")
    if indices.numel() != n_slots:
        raise ValueError("indices must have one entry per base_out row")
    p = Projection(ctypes.pointer(route), xp, x_rows, x_ld, int(bool(x_by_row)), op, out_ld,
                   _dev(indices, "indices", torch.int32),
                   _dev(row_adapter, "row_adapter", torch.int32), row_adapter.numel(),
                   n_slots, int(top_k))
    p._keep = (route, x, base_out, indices, row_adapter)
    return p


def mlora_gather_bgmv_set(projections, stream=None) -> None:
    """Gather folds of 1 to 4 projections (make_projection) in one launch."""
    arr = (Projection * len(projections))(*projections)
    rc = load().mlora_gather_bgmv_set(arr, len(projections), _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)


def mlora_resolve_moe_lora_route_multi(adapter_slot: int, n_adapters: int) -> int:
    return int(load().mlora_resolve_moe_lora_route_multi(int(adapter_slot), int(n_adapters)))


def mlora_build_moe_row_adapter_decode_multi(adapter_slots, padded_n: int,
                                             n_adapters: int) -> np.ndarray:
    sl = _arr(adapter_slots, np.int32)
    out = np.zeros(int(padded_n), dtype=np.int32)
    rc = load().mlora_build_moe_row_adapter_decode_multi(_ptr(sl, ctypes.c_int32), sl.shape[0],
                                                         int(padded_n), int(n_adapters),
                                                         _ptr(out, ctypes.c_int32))
    if rc != MLORA_OK:
        raise _err(rc)
    return out


def mlora_pack_expert_tables_multi(adapter_slots, expert_ids, a_addrs, b_addrs, scales):
    """None for no entries, else (a_table, b_table, scale_table, n_adapters,
    n_experts) with flat tables of n_adapters * n_experts cells."""
    sl = _arr(adapter_slots, np.int32)
    ids = _arr(expert_ids, np.int32)
    a = _arr(a_addrs, np.uint64)
    b = _arr(b_addrs, np.uint64)
    s = _arr(scales, np.float32)
    n = ids.shape[0]
    if not (sl.shape[0] == a.shape[0] == b.shape[0] == s.shape[0] == n):
        raise ValueError("entry arrays differ in length")
    lib = load()
    na, ne = ctypes.c_int32(0), ctypes.c_int32(0)
    args = (_ptr(sl, ctypes.c_int32), _ptr(ids, ctypes.c_int32), _ptr(a, ctypes.c_uint64),
            _ptr(b, ctypes.c_uint64), _ptr(s, ctypes.c_float), n)
    rc = lib.mlora_pack_expert_tables_multi(*args, None, None, None, 0, ctypes.byref(na),
                                            ctypes.byref(ne))
    if rc == MLORA_NONE:
        return None
    if rc != MLORA_ERR_CAPACITY:
        raise _err(rc)
    cells = na.value * ne.value
    at = np.zeros(cells, dtype=np.uint64)
    bt = np.zeros(cells, dtype=np.uint64)
    st = np.zeros(cells, dtype=np.float32)
    rc = lib.mlora_pack_expert_tables_multi(*args, _ptr(at, ctypes.c_uint64),
                                            _ptr(bt, ctypes.c_uint64), _ptr(st, ctypes.c_float),
                                            cells, ctypes.byref(na), ctypes.byref(ne))
    if rc != MLORA_OK:
        raise _err(rc)
    return at, bt, st, int(na.value), int(ne.value)


def make_multi_route(a_table, b_table, scale_table, n_adapters: int, n_experts: int, k_in: int,
                     n_out: int, max_rank: int) -> MultiRoute:
    """Multi-adapter route over device tables of n_adapters * n_experts cells
    (bf16 weights). The caller keeps the tensors alive."""
    import torch
    for t in (a_table, b_table, scale_table):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("route tables must be contiguous device tensors")
    if scale_table.dtype != torch.float32:
        raise TypeError("scale_table must be float32")
    return MultiRoute(a_table.data_ptr(), b_table.data_ptr(), scale_table.data_ptr(),
                      int(n_adapters), int(n_experts), int(k_in), int(n_out), int(max_rank),
                      MLORA_BF16)


def mlora_gather_bgmv_multi(route: MultiRoute, x, base_out, indices, row_adapter, top_k: int,
                            stream=None) -> None:
    """Multi-adapter gather fold of every flat row of ``base_out``, in place:
    row r folds with the cell (row_adapter[r // top_k], indices[r])."""
    import torch
    if x.dtype != torch.bfloat16 or base_out.dtype != torch.bfloat16:
        raise TypeError("the multi-adapter fold is bf16")
    if x.dim() != 2 or base_out.dim() != 2:
        raise ValueError("x and base_out must be 2-D")
    if x.shape[1] != route.k_in or base_out.shape[1] != route.n_out:
        raise ValueError("x / base_out widths differ from the route's k_in / n_out")
    n_slots = base_out.shape[0]
    if indices.numel() != n_slots:
        raise ValueError("indices must have one entry per base_out row")
    if row_adapter.numel() < x.shape[0]:
        raise ValueError("row_adapter must cover every x row")
    rc = load().mlora_gather_bgmv_multi(
        ctypes.byref(route), _dev(x, "x"), x.shape[0], _dev(base_out, "base_out"),
        _dev(indices, "indices", torch.int32), _dev(row_adapter, "row_adapter", torch.int32),
        n_slots, int(top_k), _stream_handle(stream))
    if rc != MLORA_OK:
        raise _err(rc)

