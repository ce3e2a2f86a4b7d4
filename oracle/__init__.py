"""CPU oracle for the streaming-reduction hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The HIP library and its Python binding never do,
and they share no code with it.

The arithmetic lives in ``loom_oracle.c`` (plain C, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only builds that file with
gcc and marshals numpy arrays into it.  See the C file for the page citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "loom_oracle.c")
_LIB = os.path.join(_HERE, "libloom_oracle.so")
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (this call builds it and runs nothing of it)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The oracle library; LOOM_ORACLE_LIB names a prebuilt copy instead (used by
    the mutation test to run the pins against an oracle with a planted mistake)."""
    global _lib
    if _lib is None:
        l = ctypes.CDLL(os.environ.get("LOOM_ORACLE_LIB") or build())
        i64, p = ctypes.c_int64, ctypes.c_void_p
        l.oracle_tile_split.argtypes = [i64, i64, p, p]
        l.oracle_fill_workgroups.argtypes = [i64, i64]
        l.oracle_fill_workgroups.restype = i64
        l.oracle_copy_f32.argtypes = [p, p, i64]
        l.oracle_row_sum_tiles.argtypes = [p, i64, p, p, p, p]
        l.oracle_row_sums.argtypes = [p, i64, i64, i64, p, p, p]
        l.oracle_segment_sums.argtypes = [p, p, i64, i64, p, p, p, p]
        l.oracle_i8_dequant_dot.argtypes = [p, p, p, p, i64, i64, i64, p, p]
        l.oracle_i8_dequant_dot.restype = ctypes.c_int
        l.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        l.oracle_f16_to_f32.restype = ctypes.c_float
        l.oracle_packed_dot.argtypes = [p, p, p, i64, p, i64, i64, p, p, p]
        l.oracle_sum_guarded_rows.argtypes = [p, i64, i64, i64, p]
        l.oracle_routed_combine.argtypes = [p, p, p, i64, i64, i64, i64, p, p, p]
        _lib = l
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _arr(a, dtype):
    a = np.ascontiguousarray(np.asarray(a), dtype=dtype)
    return a


def tile_split(count: int, tile: int = 8):
    fr, tc = ctypes.c_int64(), ctypes.c_int64()
    lib().oracle_tile_split(count, tile, ctypes.byref(fr), ctypes.byref(tc))
    return fr.value, tc.value


def fill_workgroups(element_count: int, workgroup_size: int = 256) -> int:
    return lib().oracle_fill_workgroups(element_count, workgroup_size)


def copy_f32(x):
    x = _arr(x, np.float32)
    out = np.empty_like(x)
    lib().oracle_copy_f32(_ptr(x), _ptr(out), x.size)
    return out


def row_sum_tiles(values, count: int, initial=None):
    """values [rows_alloc][32] f32 -> (sums[32] f32, final_row, tail_count)."""
    values = _arr(values, np.float32)
    assert values.ndim == 2 and values.shape[1] == 32 and 0 <= count <= values.shape[0]
    init = None if initial is None else _arr(initial, np.float32)
    sums = np.empty(32, np.float32)
    fr, tc = ctypes.c_int64(), ctypes.c_int64()
    lib().oracle_row_sum_tiles(_ptr(values), count, _ptr(init), _ptr(sums), ctypes.byref(fr), ctypes.byref(tc))
    return sums, fr.value, tc.value


def row_sums(x, shadows: bool = True):
    """x [rows][cols] f32 (row stride = cols) -> (out f32, out_f64, sum|x|) per row."""
    x = _arr(x, np.float32)
    rows, cols = x.shape
    out = np.empty(rows, np.float32)
    d = np.empty(rows, np.float64) if shadows else None
    a = np.empty(rows, np.float64) if shadows else None
    lib().oracle_row_sums(_ptr(x), rows, cols, cols, _ptr(out), _ptr(d), _ptr(a))
    return out, d, a


def segment_sums(x, offsets, shadows: bool = True):
    """x [total_rows][cols] f32, offsets int64 [S+1] -> (out [S][cols], tail_counts [S], f64, abs)."""
    x = _arr(x, np.float32)
    offsets = _arr(offsets, np.int64)
    cols = x.shape[1]
    S = offsets.size - 1
    assert offsets[0] >= 0 and offsets[-1] <= x.shape[0] and np.all(np.diff(offsets) >= 0)
    out = np.empty((S, cols), np.float32)
    tails = np.empty(S, np.int32)
    d = np.empty((S, cols), np.float64) if shadows else None
    a = np.empty((S, cols), np.float64) if shadows else None
    lib().oracle_segment_sums(_ptr(x), _ptr(offsets), S, cols, _ptr(out), _ptr(tails), _ptr(d), _ptr(a))
    return out, tails, d, a


def i8_dequant_dot(w, w_scale, x, x_scale=None):
    """w int8 [rows][k], x int8 [batch][k] -> (out f32 [rows][batch], acc int32 [rows][batch])."""
    w = _arr(w, np.int8)
    x = _arr(x, np.int8)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    rows, k = w.shape
    batch = x.shape[0]
    assert x.shape[1] == k
    ws = _arr(w_scale, np.float32)
    xs = None if x_scale is None else _arr(x_scale, np.float32)
    out = np.empty((rows, batch), np.float32)
    acc = np.empty((rows, batch), np.int32)
    st = lib().oracle_i8_dequant_dot(_ptr(w), _ptr(ws), _ptr(x), _ptr(xs), rows, k, batch, _ptr(out), _ptr(acc))
    if st != 0:
        raise OverflowError("int8 dot accumulator does not fit in int32")
    return out, acc


def f16_to_f32(bits: int) -> float:
    return lib().oracle_f16_to_f32(bits)


def packed_dot(fields, scales, rhs, count: int, initial=None, shadows: bool = True):
    """fields int32 [records][outputs], scales uint16 (binary16 bits) [records][outputs],
    rhs f32 [records][streams][4] -> (out f32 [outputs], out_f64, sum |terms|)."""
    fields = _arr(fields, np.int32)
    scales = _arr(scales, np.uint16)
    rhs = _arr(rhs, np.float32)
    records, outputs = fields.shape
    assert scales.shape == fields.shape and 0 <= count <= records
    assert rhs.ndim == 3 and rhs.shape[0] >= count and rhs.shape[2] == 4
    streams = rhs.shape[1]
    init = None if initial is None else _arr(initial, np.float32)
    out = np.empty(outputs, np.float32)
    d = np.empty(outputs, np.float64) if shadows else None
    a = np.empty(outputs, np.float64) if shadows else None
    # the oracle reads rhs rows [0, count) with the row pitch of this array
    lib().oracle_packed_dot(_ptr(fields), _ptr(scales), _ptr(rhs), streams, _ptr(init), count, outputs,
                            _ptr(out), _ptr(d), _ptr(a))
    return out, d, a


def sum_guarded_rows(values, count: int, columns: int, active_lanes: int):
    """values f32 [rows_alloc][32][4] -> sums f32 [32] (the pages' guarded ragged row sum)."""
    values = _arr(values, np.float32)
    assert values.ndim == 3 and values.shape[1:] == (32, 4) and 0 <= count <= values.shape[0]
    assert 0 <= columns <= 4 and 0 <= active_lanes <= 32
    sums = np.empty(32, np.float32)
    lib().oracle_sum_guarded_rows(_ptr(values), count, columns, active_lanes, _ptr(sums))
    return sums


def routed_combine(ids, weights, payload, shadows: bool = True):
    """ids int32 [tokens][routes], weights f32 [tokens][routes], payload f32 [num_rows][hidden]
    -> (out f32 [tokens][hidden], out_f64, sum |terms|)."""
    ids = _arr(ids, np.int32)
    weights = _arr(weights, np.float32)
    payload = _arr(payload, np.float32)
    tokens, routes = ids.shape
    num_rows, hidden = payload.shape
    assert weights.shape == ids.shape
    out = np.empty((tokens, hidden), np.float32)
    d = np.empty((tokens, hidden), np.float64) if shadows else None
    a = np.empty((tokens, hidden), np.float64) if shadows else None
    lib().oracle_routed_combine(_ptr(ids), _ptr(weights), _ptr(payload), num_rows, tokens, routes, hidden,
                                _ptr(out), _ptr(d), _ptr(a))
    return out, d, a
