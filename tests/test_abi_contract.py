"""The documented argument contract of every sized entry point, on random arguments.

Each model below restates the rules that include/loom.h gives for one entry point
(ranges, shapes, the empty call, required pointers, alignment, in the order the
header's conventions fix) and predicts the status of a call.  Arguments are drawn
at random around every documented bound, with pointers from {NULL, 16-byte
aligned, 4-byte aligned, 2-byte aligned}.  A call that passes every check would
launch, so these run only where no GPU is present: there the launch itself is
refused (LOOM_ERR_DEVICE) and no pointer is ever used.
"""
import ctypes
import os

import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

OK, NULL, RANGE, ALIGN, SHAPE, DEVICE = 0, -1, -2, -3, -4, -7
I31 = 2**31 - 1
I64 = 2**63 - 1


def _no_gpu():
    import torch
    return not torch.cuda.is_available() and not os.path.exists("/dev/kfd")


pytestmark = pytest.mark.skipif(not _no_gpu(), reason="a passing call would launch on placeholder pointers")

PTRS = st.sampled_from([None, 0x10000, 0x10004, 0x10002])
SETTINGS = settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def sizes(*bounds):
    """Integers near 0 and near each given bound, plus some in between."""
    pts = {-1, 0, 1, 2, 3, 4, 5, 7, 8}
    for b in bounds:
        pts |= {b - 1, b, b + 1}
    return st.one_of(st.sampled_from(sorted(pts)), st.integers(-2, 4096))


@pytest.fixture(scope="module")
def lib():
    import int8_dequant_dot_amd as loom
    return loom.library()


def _p(v):
    return None if v is None else ctypes.c_void_p(v)


def _status(range_or_shape, empty, null, misaligned):
    for code, hit in range_or_shape:
        if hit:
            return code
    if empty:
        return OK
    if null:
        return NULL
    if misaligned:
        return ALIGN
    return DEVICE


def _mis(p, a):
    return p is not None and p % a != 0


def _grid_refused(export, workload):
    """The header's rule for the grid limit: a workload whose launch grid would
    reach 2^32 work-items is refused with LOOM_ERR_RANGE, as the launch table
    reports it for the same workload (only evaluated when every documented
    size range holds)."""
    import int8_dequant_dot_amd as loom
    try:
        loom.launch_config_invoke(loom.launch_config_lookup(export), workload)
    except loom.LoomError as e:
        assert e.status == RANGE
        return True
    return False


@SETTINGS
@given(x=PTRS, out=PTRS, rows=sizes(I31, 2**30 - 16, 2**31 - 32), cols=sizes(I31, 768, 64), stride=sizes(I31))
def test_row_sums_contract(lib, x, out, rows, cols, stride):
    in_range = 0 <= rows <= I31 and 0 <= cols <= I31
    expect = _status([(RANGE, not in_range), (SHAPE, stride < cols),
                      (RANGE, rows > 0 and 4 * rows * stride > I64),
                      (RANGE, _grid_refused("row_sums", [rows, cols]))],
                     rows == 0, out is None or (x is None and cols > 0), _mis(x, 4) or _mis(out, 4))
    assert lib.loom_row_sums(_p(x), rows, cols, stride, _p(out), None) == expect


@SETTINGS
@given(w=PTRS, ws=PTRS, x=PTRS, xs=PTRS, out=PTRS, acc=PTRS, rows=sizes(I31, 2**26, 2**28), k=sizes(131068, 2**20),
       batch=sizes(64))
def test_i8_dequant_dot_contract(lib, w, ws, x, xs, out, acc, rows, k, batch):
    in_range = 0 <= k <= 131068 and 1 <= batch <= 64 and 0 <= rows <= I31
    expect = _status([(RANGE, not in_range), (SHAPE, k % 4 != 0),
                      (RANGE, _grid_refused("i8_dequant_dot", [rows, k, batch]))],
                     rows == 0, ws is None or out is None or (k > 0 and (w is None or x is None)),
                     any(_mis(p, 4) for p in (w, x, ws, xs, out, acc)))
    assert lib.loom_i8_dequant_dot(_p(w), _p(ws), _p(x), _p(xs), rows, k, batch, _p(out), _p(acc), None) == expect


@SETTINGS
@given(x=PTRS, off=PTRS, out=PTRS, tails=PTRS, total=sizes(2**40), segments=sizes(I31 - 1), cols=sizes(2**20),
       noalloc=st.booleans())
def test_segment_sums_contract(lib, x, off, out, tails, total, segments, cols, noalloc):
    # loom_segment_sums_noalloc has the same contract
    expect = _status([(RANGE, not (0 <= total <= 2**40 and 0 <= segments < I31 and 0 <= cols <= 2**20))],
                     segments == 0,
                     off is None or (out is None and cols > 0) or (x is None and total > 0 and cols > 0),
                     _mis(off, 8) or _mis(x, 4) or _mis(out, 4) or _mis(tails, 4))
    fn = lib.loom_segment_sums_noalloc if noalloc else lib.loom_segment_sums
    assert fn(_p(x), total, _p(off), segments, cols, _p(out), _p(tails), None) == expect


@SETTINGS
@given(f=PTRS, sc=PTRS, rhs=PTRS, init=PTRS, out=PTRS, streams=sizes(I31), records=sizes(I31, 2**40),
       count=sizes(I31), outputs=sizes(255 * I31, 2**40, 2**32 - 256, 2**34 - 1024))
def test_packed_dot_contract(lib, f, sc, rhs, init, out, streams, records, count, outputs):
    expect = _status([(RANGE, not (0 <= count <= records and count <= I31 and 0 <= outputs <= 255 * I31
                                   and 1 <= streams <= I31)),
                      (RANGE, records > 0 and 4 * records * outputs > I64),
                      (RANGE, _grid_refused("packed_dot", [outputs, count, streams]))],
                     outputs == 0, out is None or (count > 0 and (f is None or sc is None or rhs is None)),
                     _mis(f, 4) or _mis(sc, 2) or _mis(rhs, 16) or _mis(init, 4) or _mis(out, 4))
    assert lib.loom_packed_dot(_p(f), _p(sc), _p(rhs), streams, _p(init), records, count, outputs, _p(out),
                               None) == expect


@SETTINGS
@given(ids=PTRS, wts=PTRS, pay=PTRS, out=PTRS, num_rows=sizes(I31), tokens=sizes(I31), routes=sizes(2**20),
       hidden=sizes(2**20))
def test_routed_combine_contract(lib, ids, wts, pay, out, num_rows, tokens, routes, hidden):
    expect = _status([(RANGE, not (0 <= tokens <= I31 and 0 <= routes <= 2**20 and 0 <= hidden <= 2**20
                                   and 0 <= num_rows <= I31)), (SHAPE, hidden % 4 != 0)],
                     tokens == 0 or hidden == 0,
                     out is None or (routes > 0 and (ids is None or wts is None)) or (num_rows > 0 and pay is None),
                     _mis(ids, 4) or _mis(wts, 4) or _mis(pay, 16) or _mis(out, 16))
    assert lib.loom_routed_combine(_p(ids), _p(wts), _p(pay), num_rows, tokens, routes, hidden, _p(out),
                                   None) == expect


@SETTINGS
@given(inp=PTRS, out=PTRS, n=sizes(2**32 - 256, 255 * I31))
def test_copy_contract(lib, inp, out, n):
    expect = _status([(RANGE, not (0 <= n <= 2**32 - 256))], n == 0, inp is None or out is None,
                     _mis(inp, 4) or _mis(out, 4))
    assert lib.loom_copy_f32(_p(inp), _p(out), n, None) == expect
