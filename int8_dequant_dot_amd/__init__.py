"""Python binding of the MI355X streaming-reduction library (``libloom.so``).

Argument marshalling only: every step of the computation runs in the gfx950 HIP
kernels behind the C ABI declared in ``include/loom.h``.  PyTorch supplies device
memory and the stream (``torch.cuda.current_stream()``).  There is no CPU
fallback: if the HIP library is missing, importing this package raises.

Functions carry the C entry points' names without the ``loom_`` prefix.
"""
from __future__ import annotations

import ctypes
import os

import torch  # load torch's HIP runtime first so libloom.so binds to the same instance

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libloom.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib.loom_status_string.restype = ctypes.c_char_p
_lib.loom_status_string.argtypes = [ctypes.c_int]
_lib.loom_version.restype = ctypes.c_int
_lib.loom_version.argtypes = []
_lib.loom_launch_config_lookup.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_uint32)]
_lib.loom_launch_config_invoke.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint64), ctypes.c_size_t, _p]
_lib.loom_copy_f32.argtypes = [_p, _p, _i64, _p]
_lib.loom_row_sum_tiles.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _p]
_lib.loom_row_sums.argtypes = [_p, _i64, _i64, _i64, _p, _p]
_lib.loom_segment_sums.argtypes = [_p, _i64, _p, _i64, _i64, _p, _p, _p]
_lib.loom_segment_sums_noalloc.argtypes = [_p, _i64, _p, _i64, _i64, _p, _p, _p]
_lib.loom_i8_dequant_dot.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p]
_lib.loom_packed_dot.argtypes = [_p, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _p]
_lib.loom_sum_guarded_rows.argtypes = [_p, _i64, _i64, _i64, _i64, _p, _p]
_lib.loom_routed_combine.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _p, _p]
for _name in ("loom_launch_config_lookup", "loom_launch_config_invoke", "loom_copy_f32", "loom_row_sum_tiles",
              "loom_row_sums", "loom_segment_sums", "loom_segment_sums_noalloc", "loom_i8_dequant_dot",
              "loom_packed_dot",
              "loom_sum_guarded_rows", "loom_routed_combine"):
    getattr(_lib, _name).restype = ctypes.c_int

# status codes (include/loom.h)
OK, ERR_NULL, ERR_RANGE, ERR_ALIGN, ERR_SHAPE, ERR_UNKNOWN_EXPORT, ERR_TOKEN, ERR_DEVICE = 0, -1, -2, -3, -4, -5, -6, -7

EXPORTS = ("copy_f32", "row_sum_tiles", "row_sums", "segment_sums", "i8_dequant_dot", "packed_dot",
           "sum_guarded_rows", "routed_combine")


class LoomError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class LaunchConfig(ctypes.Structure):
    _fields_ = [("workgroups", ctypes.c_uint32 * 3), ("workgroup_size", ctypes.c_uint32 * 3),
                ("cluster_size", ctypes.c_uint32 * 3), ("subgroup_size", ctypes.c_uint32),
                ("workgroup_storage_bytes", ctypes.c_uint32)]

    def as_dict(self):
        return {"workgroups": tuple(self.workgroups), "workgroup_size": tuple(self.workgroup_size),
                "cluster_size": tuple(self.cluster_size), "subgroup_size": self.subgroup_size,
                "workgroup_storage_bytes": self.workgroup_storage_bytes}


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.loom_status_string(status).decode()


def version() -> int:
    return _lib.loom_version()


def _check(status: int, where: str):
    if status != OK:
        raise LoomError(status, where)


def launch_config_lookup(export_name: str) -> int:
    tok = ctypes.c_uint32()
    _check(_lib.loom_launch_config_lookup(export_name.encode(), ctypes.byref(tok)), "launch_config_lookup")
    return tok.value


def launch_config_invoke(token: int, workload) -> dict:
    vals = [int(v) & ((1 << 64) - 1) for v in workload]
    arr = (ctypes.c_uint64 * max(1, len(vals)))(*vals)
    cfg = LaunchConfig()
    _check(_lib.loom_launch_config_invoke(token, arr, len(vals), ctypes.byref(cfg)), "launch_config_invoke")
    return cfg.as_dict()


# ------------------------------------------------------------------ tensor helpers

def _target(t: torch.Tensor, name: str):
    """The current HIP device index and its current stream: the C ABI launches
    there, so every tensor must live on that device.  ``t`` (the call's first
    tensor) is checked first, so a CPU tensor is refused before any HIP call."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    device = torch.cuda.current_device()
    return device, torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, dtype, name: str, device: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.get_device() != device:
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{device}")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _buffer(t: torch.Tensor | None, dtype, numel: int, name: str, device: int, optional: bool = False):
    """A caller-supplied input or output buffer: a contiguous device tensor of `dtype` holding at
    least `numel` elements (the kernels read or write that many from its start)."""
    if t is None:
        if not optional:
            raise ValueError(f"{name} is required")
        return None
    _dev(t, dtype, name, device)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} are needed")
    return t


def copy_f32(inp: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out[i] = inp[i] for i < inp.numel(); elements of ``out`` beyond that are untouched."""
    device, stream = _target(inp, "inp")
    _dev(inp, torch.float32, "inp", device)
    _require(inp.is_contiguous(), "inp must be contiguous")
    if out is None:
        out = torch.empty_like(inp)
    _buffer(out, torch.float32, inp.numel(), "out", device)
    _check(_lib.loom_copy_f32(_ptr(inp), _ptr(out), inp.numel(), stream), "copy_f32")
    return out


def row_sum_tiles(values: torch.Tensor, count: int, initial: torch.Tensor | None = None):
    """values [rows_alloc][32] f32 -> (sums[32] f32, final_row int32[1], tail_count int32[1])."""
    device, stream = _target(values, "values")
    _dev(values, torch.float32, "values", device)
    _require(values.dim() == 2 and values.shape[1] == 32 and values.is_contiguous(),
             "values must be a contiguous [rows][32] tensor")
    _buffer(initial, torch.float32, 32, "initial", device, optional=True)
    sums = torch.empty(32, dtype=torch.float32, device=values.device)
    fr = torch.empty(1, dtype=torch.int32, device=values.device)
    tc = torch.empty(1, dtype=torch.int32, device=values.device)
    _check(_lib.loom_row_sum_tiles(_ptr(values), values.shape[0], count, _ptr(initial), _ptr(sums), _ptr(fr),
                                   _ptr(tc), stream), "row_sum_tiles")
    return sums, fr, tc


def row_sums(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """x [rows][cols] f32 with unit column stride (any row stride) -> out [rows]."""
    device, stream = _target(x, "x")
    _dev(x, torch.float32, "x", device)
    _require(x.dim() == 2 and (x.stride(1) == 1 or x.shape[1] <= 1), "x must be [rows][cols] with unit column stride")
    rows, cols = x.shape
    stride = x.stride(0) if rows > 1 else max(cols, 1)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=x.device)
    _buffer(out, torch.float32, rows, "out", device)
    _check(_lib.loom_row_sums(_ptr(x), rows, cols, stride, _ptr(out), stream), "row_sums")
    return out


def segment_sums(x: torch.Tensor, offsets: torch.Tensor, out: torch.Tensor | None = None,
                 tail_counts: torch.Tensor | None = None, want_tails: bool = True, noalloc: bool = False):
    """x [total_rows][cols] f32, offsets int64 [S+1] (CSR) -> (out [S][cols], tail_counts int32 [S]).

    noalloc=True calls loom_segment_sums_noalloc (no device allocation inside
    the call; calls that overlap on one GPU must be ordered by the caller)."""
    device, stream = _target(x, "x")
    _dev(x, torch.float32, "x", device)
    _dev(offsets, torch.int64, "offsets", device)
    _require(x.dim() == 2 and x.is_contiguous(), "x must be a contiguous [total_rows][cols] tensor")
    _require(offsets.dim() == 1 and offsets.is_contiguous() and offsets.numel() >= 1,
             "offsets must be a contiguous [segments + 1] tensor")
    S = offsets.numel() - 1
    cols = x.shape[1]
    if out is None:
        out = torch.empty(S, cols, dtype=torch.float32, device=x.device)
    _buffer(out, torch.float32, S * cols, "out", device)
    if tail_counts is None and want_tails:
        tail_counts = torch.empty(S, dtype=torch.int32, device=x.device)
    _buffer(tail_counts, torch.int32, S, "tail_counts", device, optional=True)
    fn = _lib.loom_segment_sums_noalloc if noalloc else _lib.loom_segment_sums
    _check(fn(_ptr(x), x.shape[0], _ptr(offsets), S, cols, _ptr(out), _ptr(tail_counts), stream),
           "segment_sums_noalloc" if noalloc else "segment_sums")
    return out, tail_counts


def i8_dequant_dot(w: torch.Tensor, w_scale: torch.Tensor, x: torch.Tensor, x_scale: torch.Tensor | None = None,
                   out: torch.Tensor | None = None, acc: torch.Tensor | None = None, want_acc: bool = False):
    """w int32 [rows][k/4] (packed int8), x int32 [batch][k/4] or [k/4] -> out f32 [rows][batch] (and acc)."""
    device, stream = _target(w, "w")
    _dev(w, torch.int32, "w", device)
    _dev(x, torch.int32, "x", device)
    if x.dim() == 1:
        x = x.view(1, -1)
    _require(w.dim() == 2 and w.is_contiguous(), "w must be a contiguous [rows][k/4] tensor")
    _require(x.dim() == 2 and x.is_contiguous() and x.shape[1] == w.shape[1],
             "x must be a contiguous [batch][k/4] tensor with the same k as w")
    rows, kw = w.shape
    batch = x.shape[0]
    _buffer(w_scale, torch.float32, rows, "w_scale", device)
    _buffer(x_scale, torch.float32, batch, "x_scale", device, optional=True)
    if out is None:
        out = torch.empty(rows, batch, dtype=torch.float32, device=w.device)
    _buffer(out, torch.float32, rows * batch, "out", device)
    if acc is None and want_acc:
        acc = torch.empty(rows, batch, dtype=torch.int32, device=w.device)
    _buffer(acc, torch.int32, rows * batch, "acc", device, optional=True)
    _check(_lib.loom_i8_dequant_dot(_ptr(w), _ptr(w_scale), _ptr(x), _ptr(x_scale), rows, 4 * kw, batch,
                                    _ptr(out), _ptr(acc), stream), "i8_dequant_dot")
    return (out, acc) if want_acc else out


def packed_dot(fields: torch.Tensor, scales: torch.Tensor, rhs: torch.Tensor, count: int,
               initial: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """fields int32 [records][outputs], scales int16/uint16 binary16 bits [records][outputs],
    rhs f32 [records][streams][4] -> out f32 [outputs] (the pages' ordered packed-dot recurrence)."""
    device, stream = _target(fields, "fields")
    _dev(fields, torch.int32, "fields", device)
    if scales.dtype == torch.float16:
        scales = scales.view(torch.int16)
    if scales.dtype not in (torch.int16, torch.uint16):
        raise TypeError("scales must hold binary16 bit patterns (float16, int16 or uint16)")
    _dev(scales, scales.dtype, "scales", device)
    _dev(rhs, torch.float32, "rhs", device)
    _require(fields.dim() == 2 and fields.is_contiguous(), "fields must be a contiguous [records][outputs] tensor")
    _require(scales.shape == fields.shape and scales.is_contiguous(), "scales must be contiguous, shaped as fields")
    _require(rhs.dim() == 3 and rhs.shape[2] == 4 and rhs.is_contiguous() and rhs.shape[0] >= count,
             "rhs must be a contiguous [records >= count][streams][4] tensor")
    records, outputs = fields.shape
    _buffer(initial, torch.float32, outputs, "initial", device, optional=True)
    if out is None:
        out = torch.empty(outputs, dtype=torch.float32, device=fields.device)
    _buffer(out, torch.float32, outputs, "out", device)
    _check(_lib.loom_packed_dot(_ptr(fields), _ptr(scales), _ptr(rhs), rhs.shape[1], _ptr(initial), records, count,
                                outputs, _ptr(out), stream), "packed_dot")
    return out


def sum_guarded_rows(values: torch.Tensor, count: int, columns: int, active_lanes: int,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """values f32 [rows_alloc][32][4] -> sums f32 [32] (the pages' guarded ragged row sum)."""
    device, stream = _target(values, "values")
    _dev(values, torch.float32, "values", device)
    _require(values.dim() == 3 and tuple(values.shape[1:]) == (32, 4) and values.is_contiguous(),
             "values must be a contiguous [rows][32][4] tensor")
    if out is None:
        out = torch.empty(32, dtype=torch.float32, device=values.device)
    _buffer(out, torch.float32, 32, "out", device)
    _check(_lib.loom_sum_guarded_rows(_ptr(values), values.shape[0], count, columns, active_lanes, _ptr(out),
                                      stream), "sum_guarded_rows")
    return out


def routed_combine(ids: torch.Tensor, weights: torch.Tensor, payload: torch.Tensor,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """ids int32 [tokens][routes], weights f32 [tokens][routes], payload f32 [num_rows][hidden]
    -> out f32 [tokens][hidden] (routed MoE combine; out-of-range ids are missing routes)."""
    device, stream = _target(ids, "ids")
    _dev(ids, torch.int32, "ids", device)
    _dev(weights, torch.float32, "weights", device)
    _dev(payload, torch.float32, "payload", device)
    _require(ids.dim() == 2 and ids.is_contiguous(), "ids must be a contiguous [tokens][routes] tensor")
    _require(weights.shape == ids.shape and weights.is_contiguous(), "weights must be contiguous, shaped as ids")
    _require(payload.dim() == 2 and payload.is_contiguous(), "payload must be a contiguous [rows][hidden] tensor")
    tokens, routes = ids.shape
    num_rows, hidden = payload.shape
    if out is None:
        out = torch.empty(tokens, hidden, dtype=torch.float32, device=ids.device)
    _buffer(out, torch.float32, tokens * hidden, "out", device)
    _check(_lib.loom_routed_combine(_ptr(ids), _ptr(weights), _ptr(payload), num_rows, tokens, routes, hidden,
                                    _ptr(out), stream), "routed_combine")
    return out


def pack_int8(t: torch.Tensor) -> torch.Tensor:
    """View an int8 [..., k] tensor (k % 4 == 0) as packed int32 [..., k/4] words (no copy)."""
    _require(t.dtype == torch.int8 and t.shape[-1] % 4 == 0 and t.is_contiguous(),
             "pack_int8 needs a contiguous int8 tensor whose last dimension is a multiple of 4")
    if t.shape[-1] == 0:
        return torch.empty(*t.shape[:-1], 0, dtype=torch.int32, device=t.device)
    return t.view(torch.int32)
