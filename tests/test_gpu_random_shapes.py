"""Seeded random-shape parity sweeps: every entry point against the CPU oracle
over many small shapes drawn from a fixed seed -- ragged tails, partial column
blocks, unaligned bases, strided rows, empty inputs -- on top of the
hand-picked cases in test_gpu_parity.py.  Integer results and the in-order
recurrences (segment sums, packed dot, guarded rows, routed combine, the
dequantized outputs) must match bit for bit; tree-reduced row sums within
1e-5 * sum|x| of both the oracle and its binary64 shadow.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

REL_SUM = 1e-5


@pytest.fixture(scope="module")
def loom():
    import int8_dequant_dot_amd as m
    return m


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_row_sums_random_shapes(loom, device):
    rng = np.random.default_rng(1001)
    for case in range(40):
        rows = int(rng.integers(0, 300))
        cols = int(rng.integers(0, 5000))
        pad = int(rng.choice([0, 1, 3, 64]))
        shift = int(rng.choice([0, 1]))           # 1: a base that is not 16-byte aligned
        full = synth.dense_rows(synth.DENSE.seed + case, 0, rows, cols + pad + shift)
        x = full[:, shift:shift + cols]
        g = _np(loom.row_sums(full.to(device)[:, shift:shift + cols]))
        ref, d, a = oracle.row_sums(x.contiguous().numpy())
        bound = REL_SUM * a + 1e-30
        what = (case, rows, cols, pad, shift)
        assert np.all(np.abs(g.astype(np.float64) - ref) <= bound), what
        assert np.all(np.abs(g.astype(np.float64) - d) <= bound), what


def test_row_sums_narrow_random_shapes(loom, device):
    # 1-128 columns: several rows packed into each 64-lane record
    rng = np.random.default_rng(1008)
    for case in range(40):
        rows = int(rng.integers(1, 5000))
        cols = int(rng.integers(1, 129))
        pad = int(rng.choice([0, 0, 1, 4, 7]))
        shift = int(rng.choice([0, 0, 1]))
        full = synth.dense_rows(synth.DENSE.seed + 100 + case, 0, rows, cols + pad + shift)
        x = full[:, shift:shift + cols]
        g = _np(loom.row_sums(full.to(device)[:, shift:shift + cols]))
        ref, d, a = oracle.row_sums(x.contiguous().numpy())
        bound = REL_SUM * a + 1e-30
        what = (case, rows, cols, pad, shift)
        assert np.all(np.abs(g.astype(np.float64) - ref) <= bound), what
        assert np.all(np.abs(g.astype(np.float64) - d) <= bound), what


def test_row_sum_tiles_random_shapes(loom, device):
    rng = np.random.default_rng(1002)
    for case in range(40):
        rows_alloc = int(rng.integers(0, 200))
        count = int(rng.integers(0, rows_alloc + 1))
        values = synth.normal(1000 + case, synth.S_VALUES, 0, rows_alloc * 32).view(rows_alloc, 32)
        initial = synth.normal(2000 + case, synth.S_INITIAL, 0, 32) if case % 2 else None
        sums, fr, tc = loom.row_sum_tiles(values.to(device), count,
                                          None if initial is None else initial.to(device))
        osums, ofr, otc = oracle.row_sum_tiles(values.numpy(), count,
                                               None if initial is None else initial.numpy())
        assert (int(_np(fr)[0]), int(_np(tc)[0])) == (ofr, otc) == (count - count % 8, count % 8)
        absum = np.abs(values.numpy()[:ofr]).sum() + (0 if initial is None else np.abs(initial.numpy()))
        assert np.all(np.abs(_np(sums).astype(np.float64) - osums) <= REL_SUM * absum + 1e-30), (case, count)


def test_segment_sums_random_shapes(loom, device):
    rng = np.random.default_rng(1003)
    for case in range(25):
        segments = int(rng.integers(1, 50))
        lengths = torch.from_numpy(rng.integers(0, 70, segments)).to(torch.int64)
        cols = int(rng.choice([1, 3, 4, 60, 64, 100, 256, 257, 300, 512, 600]))
        off = synth.segment_offsets(lengths)
        x = synth.segment_rows(synth.SEGMENTS.seed + case, 0, int(off[-1]), cols)
        out, tails = loom.segment_sums(x.to(device), off.to(device))
        ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
        assert np.array_equal(_bits(_np(out)), _bits(ref)), (case, cols)
        assert np.array_equal(_np(tails), rtails), case


def test_i8_dequant_dot_random_shapes(loom, device):
    rng = np.random.default_rng(1004)
    for case in range(40):
        rows = int(rng.integers(1, 200))
        k = 4 * int(rng.integers(0, 3000))
        batch = int(rng.choice([1, 1, 1, 2, 3, 7, 8, 8, 15, 16, 17, 31, 33, 64]))
        seed = 3000 + case
        w = synth.i8_rows(seed, synth.S_W, 0, rows, k)
        x = synth.i8_rows(seed, synth.S_X, 0, batch, k)
        ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
        xs = synth.scales(seed, synth.S_XSCALE, 0, batch) if case % 3 else None
        y, acc = loom.i8_dequant_dot(loom.pack_int8(w.to(device)), ws.to(device), loom.pack_int8(x.to(device)),
                                     None if xs is None else xs.to(device), want_acc=True)
        ry, racc = oracle.i8_dequant_dot(w.numpy(), ws.numpy(), x.numpy(), None if xs is None else xs.numpy())
        what = (case, rows, k, batch)
        assert np.array_equal(_np(acc), racc), what
        assert np.array_equal(_bits(_np(y)), _bits(ry)), what


def test_i8_dequant_dot_row_kernel_random_shapes(loom, device):
    # 9-16 vectors at k = 4-8 KiB: the row-streaming kernel, over tile counts
    # below and above one workgroup per CU
    rng = np.random.default_rng(1009)
    for case in range(12):
        rows = int(rng.integers(16, 4600))  # past 4096 some workgroups take two tiles
        k = 1024 * int(rng.integers(4, 9))
        batch = int(rng.integers(9, 17))
        seed = 7000 + case
        w = synth.i8_rows(seed, synth.S_W, 0, rows, k)
        x = synth.i8_rows(seed, synth.S_X, 0, batch, k)
        ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
        xs = synth.scales(seed, synth.S_XSCALE, 0, batch) if case % 2 else None
        y, acc = loom.i8_dequant_dot(loom.pack_int8(w.to(device)), ws.to(device), loom.pack_int8(x.to(device)),
                                     None if xs is None else xs.to(device), want_acc=True)
        ry, racc = oracle.i8_dequant_dot(w.numpy(), ws.numpy(), x.numpy(), None if xs is None else xs.numpy())
        what = (case, rows, k, batch)
        assert np.array_equal(_np(acc), racc), what
        assert np.array_equal(_bits(_np(y)), _bits(ry)), what


def test_i8_dequant_dot_column_kernel_random_shapes(loom, device):
    # 17-64 vectors: the column-tile kernel, over row counts that give 1 to 8
    # row tiles per wave and one or two workgroups per CU, with whole and
    # partial 256-byte records
    rng = np.random.default_rng(1011)
    for case in range(12):
        rows = int(rng.integers(1, 42000))
        k = 4 * int(rng.integers(1, 130))
        batch = int(rng.integers(17, 65))
        seed = 8000 + case
        w = synth.i8_rows(seed, synth.S_W, 0, rows, k)
        x = synth.i8_rows(seed, synth.S_X, 0, batch, k)
        ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
        xs = synth.scales(seed, synth.S_XSCALE, 0, batch) if case % 2 else None
        y, acc = loom.i8_dequant_dot(loom.pack_int8(w.to(device)), ws.to(device), loom.pack_int8(x.to(device)),
                                     None if xs is None else xs.to(device), want_acc=True)
        ry, racc = oracle.i8_dequant_dot(w.numpy(), ws.numpy(), x.numpy(), None if xs is None else xs.numpy())
        what = (case, rows, k, batch)
        assert np.array_equal(_np(acc), racc), what
        assert np.array_equal(_bits(_np(y)), _bits(ry)), what


def test_packed_dot_random_shapes(loom, device):
    rng = np.random.default_rng(1005)
    shapes = [(int(rng.integers(1, 3000)), int(rng.choice([1, 2, 3, 16, 64, 100])), int(rng.integers(0, 40)))
              for _ in range(20)]
    # large enough for several outputs per lane: stream counts dividing 64 or not
    shapes += [(65536 + 64 * 7 + 5, 64, 13), (70000, 32, 3), (65600, 48, 6), (66000, 1, 0)]
    for case, (outputs, streams, count) in enumerate(shapes):
        fields, scales, rhs, initial = synth.packed_dot_inputs(seed=4000 + case, records=count + 1, outputs=outputs,
                                                              streams=streams)
        init = initial if case % 2 else None
        g = _np(loom.packed_dot(fields.to(device), scales.to(device), rhs.to(device), count,
                                None if init is None else init.to(device)))
        ref = oracle.packed_dot(fields.numpy(), scales.numpy(), rhs.numpy(), count,
                                None if init is None else init.numpy())[0]
        assert np.array_equal(_bits(g), _bits(ref)), (case, outputs, streams, count)


def test_sum_guarded_rows_random_shapes(loom, device):
    rng = np.random.default_rng(1006)
    for case in range(40):
        rows_alloc = int(rng.integers(0, 130))
        count = int(rng.integers(0, rows_alloc + 1))
        columns = int(rng.integers(0, 5))
        active = int(rng.integers(0, 33))
        values = synth.normal(5000 + case, synth.S_VALUES, 0, rows_alloc * 128).view(rows_alloc, 32, 4)
        g = _np(loom.sum_guarded_rows(values.to(device), count, columns, active))
        ref = oracle.sum_guarded_rows(values.numpy(), count, columns, active)
        assert np.array_equal(_bits(g), _bits(ref)), (case, rows_alloc, count, columns, active)


def test_routed_combine_random_shapes(loom, device):
    rng = np.random.default_rng(1007)
    for case in range(30):
        tokens = int(rng.integers(0, 40))
        routes = int(rng.integers(0, 70))
        hidden = 4 * int(rng.integers(1, 530))
        missing = int(rng.choice([0, 10, 50, 100]))
        ids, weights, payload = synth.routed_inputs(seed=6000 + case, tokens=max(tokens, 1), routes=max(routes, 1),
                                                    hidden=hidden, missing_percent=missing)
        ids, weights = ids[:tokens, :routes].contiguous(), weights[:tokens, :routes].contiguous()
        g = _np(loom.routed_combine(ids.to(device), weights.to(device), payload.to(device)))
        ref = oracle.routed_combine(ids.numpy(), weights.numpy(), payload.numpy())[0]
        assert np.array_equal(_bits(g), _bits(ref)), (case, tokens, routes, hidden, missing)


def test_repeat_calls_are_bitwise_identical(loom, device):
    # every reduction order is fixed by the kernel's structure, not by timing:
    # repeated calls on the same inputs give the same bits
    x = synth.dense_rows(synth.DENSE.seed, 0, 3000, 4096).to(device)
    narrow = synth.dense_rows(synth.DENSE.seed, 0, 20000, 37).to(device)
    skinny = synth.dense_rows(synth.DENSE.seed, 0, 3, 1 << 20).to(device)
    lengths = torch.from_numpy(np.random.default_rng(9).integers(0, 300, 200)).to(torch.int64)
    off = synth.segment_offsets(lengths)
    seg = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), 768).to(device)
    w = loom.pack_int8(synth.i8_rows(5, synth.S_W, 0, 300, 8192).to(device))
    v8 = loom.pack_int8(synth.i8_rows(5, synth.S_X, 0, 8, 8192).to(device))
    ws = synth.scales(5, synth.S_WSCALE, 0, 300).to(device)
    runs = []
    for _ in range(2):
        runs.append([loom.row_sums(x), loom.row_sums(narrow), loom.row_sums(skinny),
                     loom.segment_sums(seg, off.to(device))[0],
                     loom.i8_dequant_dot(w, ws, v8[:1]), loom.i8_dequant_dot(w, ws, v8)])
    for a, b in zip(*runs):
        assert np.array_equal(_bits(_np(a)), _bits(_np(b)))
