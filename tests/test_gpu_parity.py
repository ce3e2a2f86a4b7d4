"""GPU parity: the gfx950 HIP path (through the C ABI) against the CPU oracle.

Gates:
  * tail counts, row indices and int32 dot accumulators: bit-exact;
  * f32 sums: |gpu - oracle| <= 1e-5 * (sum|x| + |initial|) per output, and the
    same bound against the oracle's binary64 shadow sum;
  * dequantized outputs: |gpu - oracle| <= 2e-5 * |oracle| (the epilogue is the
    same two f32 products, so in practice bit-exact);
  * segment sums: bit-exact (each column is the same in-order f32 recurrence).

Small cases span several tiles and ragged tails and are compared element by
element.  At the full workload sizes every output of the dense row sums and of
both dequant-dot workloads is compared (the inputs generated on the GPU are
copied to the host, after a regenerated sample has been checked equal to
them); the segment sums, 34 GB of input, are compared on every segment of one
sixteenth of the segments and on segments sampled from the rest.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

REL_SUM = 1e-5
REL_DQ = 2e-5


@pytest.fixture(scope="module")
def loom(device):
    import int8_dequant_dot_amd as m
    return m


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_sum_close(gpu, ref, ref64, absum, extra=0.0, what=""):
    gpu = np.asarray(gpu, np.float64)
    bound = REL_SUM * (np.asarray(absum, np.float64) + extra) + 1e-30
    err = np.abs(gpu - np.asarray(ref, np.float64))
    assert np.all(err <= bound), f"{what}: max err {err.max()} vs bound at argmax {bound.ravel()[err.argmax()]}"
    if ref64 is not None:
        err64 = np.abs(gpu - np.asarray(ref64))
        assert np.all(err64 <= bound), f"{what}: max err vs f64 {err64.max()}"


# ------------------------------------------------------------------ generator: same bits on GPU

def test_generators_identical_on_gpu(device):
    for fn, kw in [(synth.normal, {}), (synth.uniform_pm1, {}), (synth.int8_uniform, {}),
                   (synth.uniform_range, {"lo": 1e-3, "hi": 1e-2}), (synth.randint, {"lo": 0, "hi": 4096})]:
        a = fn(7, 3, 12345, 100003, device="cpu", **kw)
        b = fn(7, 3, 12345, 100003, device=device, **kw).cpu()
        assert torch.equal(a, b), fn.__name__


# ------------------------------------------------------------------ copy (launch geometry + guard)

@pytest.mark.parametrize("n", [1, 255, 256, 257, 1009, 4099, 65536 * 3 + 7])
def test_copy_f32(loom, device, n):
    x = synth.normal(synth.COPY.seed, synth.S_VALUES, 0, n)
    out = torch.full((n + 64,), -1.0, device=device)
    loom.copy_f32(x.to(device), out)
    o = _np(out)
    assert np.array_equal(o[:n].view(np.uint32), oracle.copy_f32(x.numpy()).view(np.uint32))
    assert np.all(o[n:] == -1.0)  # the over-dispatched tail stored nothing


def test_copy_page_geometry(loom, device):
    tok = loom.launch_config_lookup("copy_f32")
    assert loom.launch_config_invoke(tok, [1009])["workgroups"][0] == oracle.fill_workgroups(1009) == 4


# ------------------------------------------------------------------ tiled 32-lane row sum

def test_row_sum_tiles_iota_exhaustive(loom, device):
    # all 64 counts of a 63x32 iota tile (rows_alloc = 63) -> exact
    iota = (1 + 32 * np.arange(63)[:, None] + np.arange(32)[None, :]).astype(np.float32)
    v = torch.from_numpy(iota).to(device)
    for count in range(64):
        sums, fr, tc = loom.row_sum_tiles(v, count)
        osums, ofr, otc = oracle.row_sum_tiles(iota, count)
        assert (int(_np(fr)[0]), int(_np(tc)[0])) == (ofr, otc), count
        assert np.array_equal(_np(sums), osums), count


def test_row_sum_tiles_random_poisoned(loom, device):
    # N(0,1) tile with per-lane initial values; every row at or beyond final_row is NaN
    values, count0 = synth.tile_inputs()
    init = synth.normal(synth.TILE.seed, synth.S_INITIAL, 0, 32)
    for count in sorted({count0, 0, 1, 7, 8, 9, 15, 16, 55, 56, 63}):
        F = 8 * (count // 8)
        v = values.numpy()[:count].copy()  # exact-size allocation: rows_alloc == count
        v[F:] = np.nan
        dv = torch.from_numpy(v).to(device)
        sums, fr, tc = loom.row_sum_tiles(dv, count, init.to(device))
        osums, ofr, otc = oracle.row_sum_tiles(values.numpy(), count, init.numpy())
        assert (int(_np(fr)[0]), int(_np(tc)[0])) == (ofr, otc)
        g = _np(sums)
        assert np.all(np.isfinite(g)), count
        absum = np.abs(values.numpy()[:F]).sum()
        assert_sum_close(g, osums, None, absum, np.abs(init.numpy()), f"count {count}")


def test_row_sum_tiles_long(loom, device):
    # many tiles through the pipelined path, integer data (exact in any order)
    rows = 1000
    v = np.asarray(synth.randint(11, 0, 0, rows * 32, -8, 8).view(rows, 32), np.float32)
    for count in (999, 1000, 64, 71):
        sums, fr, tc = loom.row_sum_tiles(torch.from_numpy(v).to(device), count)
        osums, ofr, otc = oracle.row_sum_tiles(v, count)
        assert (int(_np(fr)[0]), int(_np(tc)[0])) == (ofr, otc)
        assert np.array_equal(_np(sums), osums)


# ------------------------------------------------------------------ streaming row sums

ROW_SHAPES = [(1, 1), (7, 3), (8, 256), (9, 4096), (17, 4096), (23, 1000), (33, 260), (64, 4096), (13, 4097),
              (5, 0), (3, 64), (41, 1024), (16, 8192), (70, 768), (66, 1023),
              # few long rows: a workgroup of up to 16 waves per row
              (3, 300007), (2, 1 << 20), (5, 100000), (1, 65536 + 256 * 3),
              # narrow rows: several packed into each record
              (70000, 4), (1000, 128), (999, 100), (513, 33), (65, 17), (4097, 2), (129, 64)]


@pytest.mark.parametrize("rows,cols", ROW_SHAPES)
def test_row_sums_random(loom, device, rows, cols):
    x = synth.dense_rows(synth.DENSE.seed, 0, rows, cols) if cols else torch.zeros(rows, 0)
    g = _np(loom.row_sums(x.to(device)))
    ref, d, a = oracle.row_sums(x.numpy())
    assert_sum_close(g, ref, d, a, what=f"{rows}x{cols}")


@pytest.mark.parametrize("rows,cols", [(19, 4096), (9, 37), (30, 256)])
def test_row_sums_integer_exact(loom, device, rows, cols):
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    x = (((r * 7 + c * 3) % 9) - 4).astype(np.float32)
    g = _np(loom.row_sums(torch.from_numpy(x).to(device)))
    assert np.array_equal(g, oracle.row_sums(x)[0])


@pytest.mark.parametrize("rows,cols,stride,offset", [(17, 4096, 4100, 0), (11, 300, 333, 0), (9, 256, 512, 1),
                                                     (12, 1000, 1003, 3)])
def test_row_sums_strided_poisoned(loom, device, rows, cols, stride, offset):
    # padding between rows is NaN and must never be read; an odd base offset
    # takes the 32-bit load path
    full = synth.dense_rows(synth.DENSE.seed, 0, rows, stride + offset).numpy().copy()
    full[:, :offset] = np.nan
    full[:, offset + cols:] = np.nan
    dx = torch.from_numpy(full).to(device)[:, offset:offset + cols]
    g = _np(loom.row_sums(dx))
    ref, d, a = oracle.row_sums(full[:, offset:offset + cols])
    assert_sum_close(g, ref, d, a, what="strided")


def test_row_sums_full_size(loom, device):
    rows, cols = 65536, 4096
    x = synth.dense_matrix(synth.DENSE.seed, rows, cols, device=device)
    g = _np(loom.row_sums(x))
    for r in (0, 7, 8, 40000, rows - 1):  # the GPU-generated input is the generator's
        assert torch.equal(synth.dense_rows(synth.DENSE.seed, r, 1, cols)[0], x[r].cpu())
    ref, d, a = oracle.row_sums(x.cpu().numpy())
    assert_sum_close(g, ref, d, a, what="65536x4096, every row")


# ------------------------------------------------------------------ segment sums

SEG_CASES = [
    ([0, 1, 7, 8, 9, 15, 16, 17, 0, 100, 3], 256),
    ([5, 0, 64, 13], 4),
    ([9, 31, 2], 100),        # 128-bit path, partial column block
    ([17, 8, 1], 257),        # 32-bit path (cols % 4 != 0)
    ([40, 0, 23], 512),       # two column blocks
    ([0, 0], 256),
    ([1000, 3, 511], 256),    # long segments through the steady loop
    ([3, 40, 0, 9], 1000),    # four column blocks, the last partial (128-bit path)
    ([2, 300], 2050),         # nine blocks, 32-bit path
    ([0, 5], 0),              # no columns: only the tail counts
]


@pytest.mark.parametrize("lengths,cols", SEG_CASES)
def test_segment_sums_exact(loom, device, lengths, cols):
    L = torch.tensor(lengths, dtype=torch.int64)
    off = synth.segment_offsets(L)
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), cols)
    out, tails = loom.segment_sums(x.to(device), off.to(device))
    ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
    g = _np(out)
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))  # includes +0.0 for empty segments
    assert np.array_equal(_np(tails), rtails)


@pytest.mark.parametrize("segments,max_len,cols", [(200, 3000, 256), (600, 200, 256), (250, 300, 1000),
                                                     (1100, 50, 256), (300, 64, 1000), (1500, 100, 16),
                                                     (1500, 100, 100), (1500, 100, 130)])
def test_segment_sums_ring_depths(loom, device, segments, max_len, cols):
    # the read-ahead depth follows the wave count (segments x 256-column
    # blocks: 32 rows up to 256 waves, 16 up to 1024, else 8) and the row
    # width (32 up to 64 columns, 16 up to 128); every depth gives the same
    # bits
    L = synth.segment_lengths(77, segments, max_len)
    off = synth.segment_offsets(L)
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), cols)
    out, tails = loom.segment_sums(x.to(device), off.to(device))
    ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
    assert np.array_equal(_np(out).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(_np(tails), rtails)


def test_segment_sums_page_vectors(loom, device):
    # the pages' printed column sums of the 64x32 iota, as one segment each
    from tests.golden import load as golden
    iota = (1 + 32 * np.arange(64)[:, None] + np.arange(32)[None, :]).astype(np.float32)
    cases = golden.sum_rows_iota()
    # segment i covers the first n rows of its own copy of the iota
    xs, offs = [], [0]
    for _, n, _, _ in cases:
        xs.append(iota[:n])
        offs.append(offs[-1] + n)
    xcat = np.concatenate(xs)
    out, tails = loom.segment_sums(torch.from_numpy(xcat).to(device), torch.tensor(offs, device=device))
    g = _np(out)
    for i, (case, n, offset, step) in enumerate(cases):
        assert np.array_equal(g[i], (offset + step * np.arange(32)).astype(np.float32)), case
        assert int(_np(tails)[i]) == n % 8


def test_segment_sums_bad_offsets_reported(loom, device):
    x = torch.ones(10, 8, device=device)
    off = torch.tensor([0, 4, 3, 12, 12], device=device)  # decreasing, then beyond total_rows
    out, tails = loom.segment_sums(x, off)
    g, t = _np(out), _np(tails)
    assert np.all(g[0] == 4.0) and np.all(np.isnan(g[1])) and np.all(np.isnan(g[2]))
    assert list(t) == [4, -1, -1, -1]
    assert np.all(np.isnan(g[3]))  # [12, 12) lies beyond the 10 rows


# Few long segments: fewer than 1024 segment waves and at least 1024 rows per
# segment on average split every segment into P parts, each summed in row
# order, and add the part sums in part order (a fixed order: the same bits
# on every call, within the f32 tolerance of the in-order sums).
SPLIT_CASES = [
    ([100000], 256),                      # one segment, 195 parts
    ([40000, 0, 35000], 256),             # an empty segment among long ones
    ([3000, 50000, 7, 20000], 1000),      # four column blocks, a 7-row segment with mostly empty parts
    ([60000, 12345], 257),                # 32-bit path (cols % 4 != 0), two blocks
    ([30000, 30000], 100),                # one partial block
]


def _parts(loom, segments, cols, total):
    # one wave per part, whether a part's wave has a workgroup to itself or
    # sits in a run of parts
    cfg = loom.launch_config_invoke(loom.launch_config_lookup("segment_sums"), [segments, cols, total])
    return cfg["workgroups"][0] * (cfg["workgroup_size"][0] // 64) // segments


def _runs(loom, segments, cols, total):
    # the parts go in runs, a multi-wave workgroup per run
    cfg = loom.launch_config_invoke(loom.launch_config_lookup("segment_sums"), [segments, cols, total])
    return cfg["workgroup_size"][0] > 64


@pytest.mark.parametrize("lengths,cols", SPLIT_CASES)
def test_segment_sums_split_within_tolerance(loom, device, lengths, cols):
    L = torch.tensor(lengths, dtype=torch.int64)
    off = synth.segment_offsets(L)
    total = int(off[-1])
    assert _parts(loom, len(lengths), cols, total) > 1
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
    dx, doff = x.to(device), off.to(device)
    out, tails = loom.segment_sums(dx, doff)
    g = _np(out)
    ref, rtails, d, a = oracle.segment_sums(x.numpy(), off.numpy())
    assert_sum_close(g, ref, d, a, what=f"split {lengths}x{cols}")
    assert np.array_equal(_np(tails), rtails)
    assert np.array_equal(g[L.numpy() == 0].view(np.uint32), ref[L.numpy() == 0].view(np.uint32))  # +0.0
    again, _ = loom.segment_sums(dx, doff)
    assert np.array_equal(_np(again).view(np.uint32), g.view(np.uint32))  # the same bits on every call


def test_segment_sums_split_integer_exact(loom, device):
    # small integers: every partial and every sum is exact in f32, so the split
    # sums equal the in-order recurrence bit for bit
    lengths, cols = [70000, 3, 41000], 256
    L = torch.tensor(lengths, dtype=torch.int64)
    off = synth.segment_offsets(L)
    total = int(off[-1])
    assert _parts(loom, 3, cols, total) > 1
    x = (synth.randint(93, 1, 0, total * cols, -8, 8).view(total, cols)).to(torch.float32)
    out, tails = loom.segment_sums(x.to(device), off.to(device))
    ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
    assert np.array_equal(_np(out).view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(_np(tails), rtails)


def test_segment_sums_split_bad_offsets(loom, device):
    total, cols = 90000, 256
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
    off = torch.tensor([0, 40000, 30000, 90000, 90001], dtype=torch.int64)  # decreasing, then past the rows
    assert _parts(loom, 4, cols, total) > 1
    out, tails = loom.segment_sums(x.to(device), off.to(device))
    g, t = _np(out), _np(tails)
    ref, _, d, a = oracle.segment_sums(x.numpy()[:40000], np.array([0, 40000]))
    assert_sum_close(g[0], ref[0], d[0], a[0], what="split segment before bad ones")
    assert np.all(np.isnan(g[1])) and np.all(np.isnan(g[3]))
    ref2, _, d2, a2 = oracle.segment_sums(x.numpy()[30000:90000], np.array([0, 60000]))
    assert_sum_close(g[2], ref2[0], d2[0], a2[0], what="split segment after a bad one")
    assert list(t) == [0, -1, 0, -1]


# Many long segments of uneven length (2 to 2^15 segments averaging at least
# 512 rows, at least 2^26 floats, not split) are first sorted by length so the
# waves take them longest first: only the dispatch order changes, so every
# output is still the in-order recurrence bit for bit.
ORDER_CASES = [
    (300, 1600, 256, [40000, 0, 17]),     # a long head, an empty and a short segment
    (100, 1400, 1000, [30000, 1, 2]),     # four column blocks
    (200, 2600, 256, [60000, 0]),         # 200 waves: just too many to split
]


def _ordered(loom, segments, cols, total):
    return (2 <= segments <= 2 ** 15 and total // segments >= 512 and total * cols >= 2 ** 26
            and _parts(loom, segments, cols, total) == 1)


@pytest.mark.parametrize("segments,max_len,cols,head", ORDER_CASES)
def test_segment_sums_longest_first_exact(loom, device, segments, max_len, cols, head):
    tail = synth.segment_lengths(78, segments - len(head), max_len)
    L = torch.cat([torch.tensor(head, dtype=torch.int64), tail])
    off = synth.segment_offsets(L)
    total = int(off[-1])
    assert _ordered(loom, segments, cols, total)
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
    dx, doff = x.to(device), off.to(device)
    ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
    for noalloc in (False, True):
        out, tails = loom.segment_sums(dx, doff, noalloc=noalloc)
        assert np.array_equal(_np(out).view(np.uint32), ref.view(np.uint32)), noalloc
        assert np.array_equal(_np(tails), rtails), noalloc


def test_segment_sums_longest_first_bad_offsets(loom, device):
    S, cols = 400, 256
    L = synth.segment_lengths(79, S, 1400)
    off = synth.segment_offsets(L)
    total = int(off[-1])
    assert _ordered(loom, S, cols, total)
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
    bad = off.clone()
    bad[10], bad[300] = bad[11] + 5, total + 3   # segment 9 ends past segment 10's end; 299 and 300 leave the rows
    out, tails = loom.segment_sums(x.to(device), bad.to(device))
    g, t = _np(out), _np(tails)
    ok = np.ones(S, bool)
    ok[[10, 299, 300]] = False        # decreasing [bad[10], bad[11]) and both ends past total_rows
    ref, rtails, _, _ = oracle.segment_sums(x.numpy(), off.numpy())
    assert np.all(np.isnan(g[~ok])) and np.all(t[~ok] == -1)
    keep = np.flatnonzero(ok)
    keep = keep[keep != 9]            # segment 9 now reads [off[9], off[11] + 5)
    assert np.array_equal(g[keep].view(np.uint32), ref[keep].view(np.uint32))
    assert np.array_equal(t[keep], rtails[keep])
    b9, e9 = int(off[9]), int(off[11]) + 5
    r9, rt9, _, _ = oracle.segment_sums(x.numpy()[b9:e9], np.array([0, e9 - b9]))
    assert np.array_equal(g[9].view(np.uint32), r9[0].view(np.uint32)) and t[9] == rt9[0]


def _alternating(segments, short, long, extra=()):
    L = torch.tensor([short, long] * (segments // 2) + list(extra), dtype=torch.int64)
    return L


# Both sides of every threshold that picks a segment-sum launch form: the
# split reading (fewer than 192 waves and at least 1024 rows per segment on
# average) and longest-first order (2 to 2^15 segments, at least 512 rows on
# average, at least 2^26 floats).  Split launches are checked within the f32
# tolerance and for the same bits on a second call; every other launch is the
# in-order recurrence bit for bit.
BOUNDARY_CASES = [
    ("split", lambda: torch.full((191,), 1100, dtype=torch.int64), 256),        # 191 waves
    ("in_order", lambda: torch.full((192,), 1100, dtype=torch.int64), 256),     # 192 waves
    ("split", lambda: torch.full((8,), 1024, dtype=torch.int64), 256),          # 1024 rows on average
    ("in_order", lambda: torch.full((8,), 1023, dtype=torch.int64), 256),       # 1023
    ("in_order", lambda: _alternating(2 ** 15, 256, 768), 4),                   # 2^15 segments: longest first
    ("in_order", lambda: _alternating(2 ** 15, 256, 768, [512]), 4),            # 2^15 + 1: index order
    ("in_order", lambda: _alternating(4096, 254, 768), 64),                     # 511 rows on average
    ("in_order", lambda: _alternating(4096, 256, 768), 64),                     # 512
    ("in_order", lambda: _alternating(4096, 256, 768), 31),                     # 2^26 - 2^21 floats
    ("in_order", lambda: _alternating(4096, 256, 768), 32),                     # 2^26
    ("split", lambda: torch.full((1,), 15 * 512, dtype=torch.int64), 256),      # 15 parts: one partial per part
    ("runs", lambda: torch.full((1,), 16 * 512, dtype=torch.int64), 256),       # 16 parts: 2 runs of 8
    ("runs", lambda: torch.full((2,), 31 * 512, dtype=torch.int64), 512),       # 31 -> 24 parts, 512 columns
    ("split", lambda: torch.full((2,), 31 * 512, dtype=torch.int64), 513),      # 513 columns: no runs
    ("runs", lambda: torch.tensor([40 * 512 + 77, 9 * 512], dtype=torch.int64), 3),  # 32-bit path, ragged
]


@pytest.mark.parametrize("form,lengths,cols", BOUNDARY_CASES,
                         ids=[f"{i}-{c[0]}-{c[2]}cols" for i, c in enumerate(BOUNDARY_CASES)])
def test_segment_sums_form_boundaries(loom, device, form, lengths, cols):
    L = lengths()
    off = synth.segment_offsets(L)
    total = int(off[-1])
    S = L.numel()
    assert (_parts(loom, S, cols, total) > 1) == (form != "in_order")
    assert _runs(loom, S, cols, total) == (form == "runs")
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
    dx, doff = x.to(device), off.to(device)
    out, tails = loom.segment_sums(dx, doff)
    g = _np(out)
    ref, rtails, d, a = oracle.segment_sums(x.numpy(), off.numpy())
    assert np.array_equal(_np(tails), rtails)
    if form != "in_order":
        assert_sum_close(g, ref, d, a, what=f"split boundary {S}x{cols}")
        again, _ = loom.segment_sums(dx, doff)
        assert np.array_equal(_np(again).view(np.uint32), g.view(np.uint32))
    else:
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


def test_segment_sums_full_size(loom, device):
    S, cols = 16384, 256
    L = synth.segment_lengths(synth.SEGMENTS.seed, S, 4096)
    off = synth.segment_offsets(L)
    total = int(off[-1])
    x = synth.segment_matrix(synth.SEGMENTS.seed, total, cols, device=device)
    out, tails = loom.segment_sums(x, off.to(device))
    g, t = _np(out), _np(tails)
    assert np.array_equal(t, (L.numpy() % 8).astype(np.int32))
    # every segment of one sixteenth (1024 consecutive segments, ~2 GB of rows)
    s0, s1 = 5 * S // 16, 6 * S // 16
    b, e = int(off[s0]), int(off[s1])
    assert torch.equal(synth.segment_rows(synth.SEGMENTS.seed, b, 1, cols)[0], x[b].cpu())
    ref, _, _, _ = oracle.segment_sums(x[b:e].cpu().numpy(), (off[s0:s1 + 1] - b).numpy())
    assert np.array_equal(g[s0:s1].view(np.uint32), ref.view(np.uint32))
    # and segments sampled from the rest, their rows regenerated on the host
    rng = np.random.default_rng(1)
    longest = int(L.argmax())
    sample = np.unique(np.concatenate([[0, S - 1, longest], np.flatnonzero(L.numpy() == 0)[:2],
                                       rng.integers(0, S, 24)]))
    del x
    torch.cuda.empty_cache()
    for s in sample:
        b, e = int(off[s]), int(off[s + 1])
        xs = synth.segment_rows(synth.SEGMENTS.seed, b, e - b, cols)
        ref, _, _, _ = oracle.segment_sums(xs.numpy(), np.array([0, e - b]))
        assert np.array_equal(g[s].view(np.uint32), ref[0].view(np.uint32)), s


# ------------------------------------------------------------------ int8 dequant dot

def _i8_case(seed, rows, k, batch, with_xscale=True):
    w = synth.i8_rows(seed, synth.S_W, 0, rows, k)
    x = synth.i8_rows(seed, synth.S_X, 0, batch, k)
    ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
    xs = synth.scales(seed, synth.S_XSCALE, 0, batch) if with_xscale else None
    return w, x, ws, xs


def _run_i8(loom, device, w, x, ws, xs):
    y, acc = loom.i8_dequant_dot(loom.pack_int8(w.to(device)), ws.to(device), loom.pack_int8(x.to(device)),
                                 None if xs is None else xs.to(device), want_acc=True)
    return _np(y), _np(acc)


def _check_i8(gy, gacc, w, x, ws, xs, what):
    ry, racc = oracle.i8_dequant_dot(w.numpy(), ws.numpy(), x.numpy(), None if xs is None else xs.numpy())
    assert np.array_equal(gacc, racc), f"{what}: acc mismatch"
    err = np.abs(gy.astype(np.float64) - ry)
    assert np.all(err <= REL_DQ * np.abs(ry)), f"{what}: max rel err {np.max(err / np.maximum(np.abs(ry), 1e-30))}"


I8_CASES = [
    # (rows, k, batch) -- batch 1 runs a v_dot4 GEMV, batch >= 2 an MFMA kernel.
    # One vector, rows of up to 512 bytes packed several to a record (1 to 32
    # lanes per row; a wave per 64 rows; groups partly past the row):
    (1, 4, 1), (7, 4, 1), (5, 0, 1), (100, 8, 1), (65, 16, 1), (130, 20, 1), (64, 64, 1), (200, 100, 1),
    (129, 252, 1), (1000, 256, 1), (77, 260, 1), (300, 508, 1), (4097, 512, 1),
    # rows of whole 1 KiB records, a wave per block of rows (blocks that end
    # mid-matrix), or a workgroup per row at k = 8192:
    (8, 1024, 1), (70, 3072, 1), (13, 4096, 1), (17, 8192, 1), (5, 16384, 1),
    # other rows longer than 512 bytes in groups of rows per record: 4 rows x
    # 256 B pieces (partial last pieces when k is not a multiple of 256) or 2
    # rows x 512 B, groups and waves that end mid-matrix
    (3, 516, 1), (200, 528, 1), (200, 768, 1), (9, 1028, 1), (33, 1040, 1), (77, 1280, 1), (100, 2112, 1),
    (3000, 1536, 1), (257, 2560, 1), (41, 4092, 1), (19, 4100, 1), (130, 4608, 1), (23, 5124, 1),
    (5, 8704, 1), (40, 12804, 1), (6, 16896, 1),
    # both sides of each form's edge: the wide form at 6 and 7 KiB (5 KiB and
    # 9 KiB rows walk row by row), the grouped form up to 12284 bytes (12288
    # is whole records)
    (33, 6144, 1), (21, 7168, 1), (12, 5120, 1), (3, 9216, 1), (9, 12284, 1), (10, 12288, 1),
    # rows of 3 to 12 KiB that are a multiple of 16 but not of 1024 bytes: a
    # workgroup per row whose last record is partly empty (2 to 6 waves), next
    # to the grouped form just below (3056) and the row form at 12288
    (20, 3088, 1), (7, 3056, 1), (33, 4608, 1), (1, 5632, 1), (50, 8704, 1), (7, 11008, 1), (11, 12272, 1),
    (3, 64, 2), (15, 256, 3), (16, 260, 8), (17, 1000, 8), (100, 8192, 8), (33, 64, 16), (40, 512, 17),
    (20, 1024, 32), (18, 320, 33), (16, 4096, 64), (1, 4, 2), (31, 8, 5),
    # the tile kernel's k split: 1 wave per tile (k <= 2048, several records),
    # 2 (k = 4096), 4 (k = 16384 with few tiles, k = 32768) and 8 (k = 16384,
    # 513 tiles)
    (1000, 2048, 7), (100, 4096, 8), (300, 16384, 8), (50, 32768, 2), (8200, 16384, 3),
    # the tile kernel and the row kernel with a single row, partial last
    # tiles and thousands of tiles
    (1, 2048, 2), (4111, 8192, 5), (12345, 6144, 15), (40000, 2048, 2), (333, 4096, 3),
    # 7-8 vectors, and 2-8 vectors when 8 waves split k: the segment-paired
    # kernel (A operand = 4 rows x 4 k segments, no LDS staging); one and two
    # vector groups, ragged tiles, partial last records, 1 to 8 waves per tile;
    # 6 vectors on the tile kernel next to it
    (13, 8192, 7), (70, 1024, 7), (33, 256, 7), (8200, 16384, 8), (8193, 16384, 2), (8300, 16384, 4),
    (8210, 16388, 5), (600, 16384, 7), (13, 8192, 6), (8200, 16384, 6),
    # 8 waves per tile with 3 vectors and a partly empty last record (k a
    # multiple of 16, not of 256), with 7 vectors at whole records, and one
    # whole 16-row tile
    (8197, 20000, 3), (8240, 16640, 7), (16, 8192, 8),
    # 9-16 vectors with k a multiple of 1024 from 4096 to 8192: the row-streaming
    # kernel (one workgroup per CU walking 16-row tiles; 8197 rows give 513
    # tiles, so workgroups take two or three tiles each)
    (16, 4096, 9), (17, 4096, 16), (100, 6144, 12), (300, 8192, 16), (47, 5120, 11), (8197, 4096, 16),
    (1000, 7168, 13),
    # more than 16 vectors: 64-row workgroups, one wave per 16-vector column
    # tile and row group; partial records, partial tiles, a workgroup with
    # fewer than 16 rows, exactly one and a few full workgroups
    (33, 8192, 48), (17, 1000, 20), (50, 260, 64), (300, 4096, 40),
    (5, 2048, 64), (64, 8192, 64), (65, 1024, 33), (192, 2048, 32), (129, 8192, 17),
    # workgroups start their k walk at different records, wrapping around, also
    # at a partial last record
    (200, 1000, 40), (150, 260, 64), (260, 4100, 24),
    # four column tiles: 1 to 8 row tiles per wave (rows shared evenly by one or
    # two workgroups per CU), the last workgroup partial
    (5000, 512, 64), (12000, 260, 40), (16384, 256, 33), (20000, 128, 64), (24576, 256, 40),
    (24600, 1000, 64), (30000, 64, 48), (40000, 64, 64),
]


@pytest.mark.parametrize("rows,k,batch", I8_CASES)
def test_i8_dequant_dot(loom, device, rows, k, batch):
    w, x, ws, xs = _i8_case(100 + rows + k + batch, rows, k, batch, with_xscale=(batch % 2 == 0))
    gy, gacc = _run_i8(loom, device, w, x, ws, xs)
    _check_i8(gy, gacc, w, x, ws, xs, f"{rows}x{k}x{batch}")


@pytest.mark.parametrize("rows,k,batch", [(70, 4096, 8), (70, 4096, 16), (70, 4096, 33), (70, 4096, 1),
                                           (4111, 8192, 5), (90, 2048, 2), (70, 6144, 12),
                                           (70, 8192, 1), (70, 7168, 1), (70, 6144, 1), (70, 5000, 1),
                                           (70, 4608, 1), (70, 11008, 1),
                                           (70, 1536, 1), (70, 1028, 1),
                                           (130, 100, 1), (130, 12, 1)])
def test_i8_unaligned_operands(loom, device, rows, k, batch):
    # weights and vectors starting 4 bytes past a 16-byte boundary: the kernels
    # read them as single words instead of 16-byte groups (for one vector in
    # each GEMV form)
    w, x, ws, xs = _i8_case(77 + batch + k, rows, k, batch)
    wbuf = torch.zeros(rows * k // 4 + 1, dtype=torch.int32, device=device)
    xbuf = torch.zeros(batch * k // 4 + 1, dtype=torch.int32, device=device)
    wp = wbuf[1:].view(rows, k // 4)
    xp = xbuf[1:].view(batch, k // 4)
    wp.copy_(loom.pack_int8(w.to(device)))
    xp.copy_(loom.pack_int8(x.to(device)))
    assert wp.data_ptr() % 16 == 4 and xp.data_ptr() % 16 == 4
    y, acc = loom.i8_dequant_dot(wp, ws.to(device), xp, xs.to(device), want_acc=True)
    _check_i8(_np(y), _np(acc), w, x, ws, xs, f"unaligned {rows}x{k}x{batch}")


@pytest.mark.parametrize("batch", [1, 2, 8, 16, 64])
def test_i8_extremes_at_int32_limit(loom, device, batch):
    # k = 131068 with every byte -128: acc = 16384 k = 2^31 - 65536, the largest
    # accumulator the range check admits; the opposite sign on half the vectors
    # (one vector: the GEMV; 2 and 16: the tile kernel; 8: the segment-paired
    # kernel; 64: the column-tile kernel)
    k, rows = 131068, 17
    w = torch.full((rows, k), -128, dtype=torch.int8)
    x = torch.full((batch, k), -128, dtype=torch.int8)
    x[1::2] = 127
    ws = torch.ones(rows)
    xs = torch.ones(batch) if batch > 1 else None
    gy, gacc = _run_i8(loom, device, w, x, ws, xs)
    assert gacc[0, 0] == 16384 * k
    if batch > 1:
        assert gacc[0, 1] == -16256 * k
    _check_i8(gy, gacc, w, x, ws, xs, "extremes")


def test_i8_one_hot_and_byte_order(loom, device):
    # one-hot activations pick single weight columns: pins byte order and
    # sign extension through the packed words on every kernel (one vector: the
    # GEMV; 2 and 16: the tile kernel; 8: the segment-paired kernel; 64: the
    # column-tile kernel)
    rows, k = 24, 256
    w = synth.i8_rows(5, synth.S_W, 0, rows, k)
    for batch in (1, 2, 8, 16, 64):
        cols = ([3, 64, 129, 255, 0, 17, 18, 19] + [(37 * b + 5) % k for b in range(8, 64)])[:batch]
        x = torch.zeros(batch, k, dtype=torch.int8)
        for b, c in enumerate(cols):
            x[b, c] = 1
        gy, gacc = _run_i8(loom, device, w, x, torch.ones(rows), None)
        assert np.array_equal(gacc, w.numpy()[:, cols].astype(np.int32))


def _i8_full(loom, device, wl, rows, k, batch):
    seed = wl.seed
    w = synth.i8_matrix(seed, synth.S_W, rows, k, device=device)
    x = synth.i8_matrix(seed, synth.S_X, batch, k, device=device)
    ws = synth.scales(seed, synth.S_WSCALE, 0, rows, device=device)
    xs = synth.scales(seed, synth.S_XSCALE, 0, batch, device=device) if batch > 1 else None
    y, acc = loom.i8_dequant_dot(loom.pack_int8(w), ws, loom.pack_int8(x), xs, want_acc=True)
    gy, gacc = _np(y), _np(acc)
    rng = np.random.default_rng(2)
    sample = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 48)]))
    wsamp = torch.cat([synth.i8_rows(seed, synth.S_W, int(r), 1, k) for r in sample])
    assert torch.equal(wsamp[0].to(device), w[int(sample[0])])
    xcpu = synth.i8_rows(seed, synth.S_X, 0, batch, k)
    wscpu = synth.scales(seed, synth.S_WSCALE, 0, rows)[torch.from_numpy(sample)]
    xscpu = synth.scales(seed, synth.S_XSCALE, 0, batch) if batch > 1 else None
    _check_i8(gy[sample], gacc[sample], wsamp, xcpu, wscpu, xscpu, f"{rows}x{k}x{batch} sampled")
    # every output, against the oracle over row blocks on the host cores (each
    # output's arithmetic is the single-threaded oracle's)
    from concurrent.futures import ThreadPoolExecutor
    hw, hx, hws = w.cpu().numpy(), x.cpu().numpy(), ws.cpu().numpy()
    hxs = None if xs is None else xs.cpu().numpy()
    blocks = [(a, min(rows, a + 2048)) for a in range(0, rows, 2048)]
    with ThreadPoolExecutor(min(16, len(blocks))) as pool:
        parts = list(pool.map(lambda ab: oracle.i8_dequant_dot(hw[ab[0]:ab[1]], hws[ab[0]:ab[1]], hx, hxs), blocks))
    ry = np.concatenate([p[0] for p in parts])
    racc = np.concatenate([p[1] for p in parts])
    assert np.array_equal(gacc, racc.reshape(gacc.shape)), f"{rows}x{k}x{batch}: acc mismatch"
    err = np.abs(gy.astype(np.float64) - ry.reshape(gy.shape))
    assert np.all(err <= REL_DQ * np.abs(ry.reshape(gy.shape))), f"{rows}x{k}x{batch}: max err {err.max()}"


def test_i8_gemv_full_size(loom, device):
    _i8_full(loom, device, synth.GEMV, 16384, 8192, 1)


def test_i8_batched_full_size(loom, device):
    _i8_full(loom, device, synth.BATCHED, 28672, 8192, 8)


@pytest.mark.parametrize("rows,k", [(28672, 8192), (57344, 4096)])
def test_i8_batched_64_full_size(loom, device, rows, k):
    # the column-tile kernel at full size: one (7 row tiles per wave) and two
    # workgroups per CU
    _i8_full(loom, device, synth.BATCHED, rows, k, 64)


def test_tile_workload(loom, device):
    # the pages' own tile: one 63x32 N(0,1) tile, seeded count
    values, count = synth.tile_inputs()
    sums, fr, tc = loom.row_sum_tiles(values.to(device), count)
    osums, ofr, otc = oracle.row_sum_tiles(values.numpy(), count)
    assert (int(_np(fr)[0]), int(_np(tc)[0])) == (ofr, otc)
    assert_sum_close(_np(sums), osums, None, np.abs(values.numpy()[:ofr]).sum(), what="tile")


# ------------------------------------------------------------------ packed dot (pages' literal form)

PACKED_LENGTHS = [0, 1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 127, 128]  # 14 lengths, as on the page


def _run_packed(loom, device, fields, scales, rhs, count, initial):
    out = loom.packed_dot(fields.to(device), scales.to(device), rhs.to(device), count,
                          None if initial is None else initial.to(device))
    return _np(out)


@pytest.mark.parametrize("count", PACKED_LENGTHS)
def test_packed_dot_page_shape_bitwise(loom, device, count):
    # 2048 outputs x up to 128 records, 64 shared streams: the GPU recurrence
    # must equal the serial oracle bit for bit at every length
    fields, scales, rhs, initial = synth.packed_dot_inputs()
    g = _run_packed(loom, device, fields, scales, rhs, count, initial)
    ref = oracle.packed_dot(fields.numpy(), scales.numpy(), rhs.numpy(), count, initial.numpy())[0]
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("outputs,streams,count", [(1, 1, 5), (100, 3, 17), (70001, 64, 9), (300, 100, 33),
                                                   (64, 64, 128),
                                                   # several outputs per lane, a ragged last wave
                                                   (65536 + 37, 1, 6), (65536 + 1000, 16, 11), (66560, 32, 21),
                                                   # 128 streams do not divide the wave: one output per lane
                                                   (65536, 128, 7)])
def test_packed_dot_odd_shapes_bitwise(loom, device, outputs, streams, count):
    fields, scales, rhs, initial = synth.packed_dot_inputs(seed=70 + outputs, records=max(count, 1) + 2,
                                                          outputs=outputs, streams=streams)
    for init in (initial, None):
        g = _run_packed(loom, device, fields, scales, rhs, count, init)
        ref = oracle.packed_dot(fields.numpy(), scales.numpy(), rhs.numpy(), count,
                                None if init is None else init.numpy())[0]
        assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


def test_packed_dot_large_sampled(loom, device):
    records, outputs, streams = 128, 262144, 64
    fields, scales, rhs, initial = synth.packed_dot_inputs(seed=77, records=records, outputs=outputs,
                                                          streams=streams, device=device)
    g = _np(loom.packed_dot(fields, scales, rhs, records, initial))
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, outputs - 1], rng.integers(0, outputs, 200)]))
    f, s, r, i = (t.cpu().numpy() for t in (fields, scales, rhs, initial))
    # each sampled output keeps its own activation stream (o mod 64)
    ref = np.array([oracle.packed_dot(f[:, [o]], s[:, [o]], r[:, [o % streams]], records, i[[o]])[0][0]
                    for o in sample], np.float32)
    assert np.array_equal(g[sample].view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ guarded ragged rows (pages' motif)

def test_sum_guarded_rows_360_combinations_bitwise(loom, device):
    # mixed-sign inputs, bit for bit, across 6 row counts x 5 inner extents x
    # 4 active-lane counts x 3 seeds = 360 combinations; each allocation ends
    # at `count` rows, so the padded row never exists
    n = 0
    for seed in (1, 2, 3):
        full = synth.normal(seed, synth.S_VALUES, 0, 63 * 32 * 4).view(63, 32, 4)
        for count in (0, 1, 3, 4, 5, 63):
            v = full[:count].contiguous()
            dv = v.to(device) if count else torch.zeros((0, 32, 4), device=device)
            for columns in range(5):
                for active in (0, 1, 17, 32):
                    g = _np(loom.sum_guarded_rows(dv, count, columns, active))
                    ref = oracle.sum_guarded_rows(full.numpy(), count, columns, active)
                    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32)), (seed, count, columns, active)
                    n += 1
    assert n == 360


def test_sum_guarded_rows_poisoned(loom, device):
    # NaN in every element the guards exclude must not reach the sums
    v = synth.normal(9, synth.S_VALUES, 0, 63 * 32 * 4).view(63, 32, 4).numpy().copy()
    for count, columns, active in [(63, 2, 17), (5, 3, 31), (62, 1, 1)]:
        p = v.copy()
        p[count:] = np.nan
        p[:, active:] = np.nan
        p[:, :, columns:] = np.nan
        g = _np(loom.sum_guarded_rows(torch.from_numpy(p).to(device), count, columns, active))
        assert np.array_equal(g.view(np.uint32), oracle.sum_guarded_rows(v, count, columns, active).view(np.uint32))


# ------------------------------------------------------------------ routed row combine

def _run_routed(loom, device, ids, weights, payload):
    return _np(loom.routed_combine(ids.to(device), weights.to(device), payload.to(device)))


@pytest.mark.parametrize("tokens,routes", [(1, 8), (16, 8), (256, 8), (1, 32), (16, 32), (256, 32)])
def test_routed_combine_page_shapes_bitwise(loom, device, tokens, routes):
    # the pages' n8/n32 x t1/t16/t256 workloads, 1024-wide rows, 5% missing routes
    ids, weights, payload = synth.routed_inputs(seed=80 + tokens + routes, tokens=tokens, routes=routes)
    g = _run_routed(loom, device, ids, weights, payload)
    ref = oracle.routed_combine(ids.numpy(), weights.numpy(), payload.numpy())[0]
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("tokens,routes,hidden,missing", [(3, 0, 64, 5), (5, 100, 260, 20), (2, 64, 4, 50),
                                                          (9, 65, 512, 5), (4, 7, 1024, 100), (1, 130, 8, 0),
                                                          (3, 9, 2052, 10)])
def test_routed_combine_edges_bitwise(loom, device, tokens, routes, hidden, missing):
    ids, weights, payload = synth.routed_inputs(seed=90 + routes, tokens=tokens, routes=max(routes, 1),
                                                hidden=hidden, missing_percent=missing)
    ids, weights = ids[:, :routes].contiguous(), weights[:, :routes].contiguous()
    w = weights.clone()
    w[(ids < 0) | (ids >= payload.shape[0])] = float("nan")   # weights of missing routes are never read
    g = _run_routed(loom, device, ids, w, payload)
    ref = oracle.routed_combine(ids.numpy(), weights.numpy(), payload.numpy())[0]
    assert np.array_equal(g.view(np.uint32), ref.view(np.uint32))


def test_routed_combine_no_rows(loom, device):
    ids = torch.tensor([[0, 1, -1]], dtype=torch.int32)
    g = _run_routed(loom, device, ids, torch.ones(1, 3), torch.zeros(0, 16))
    assert np.all(g == 0) and not np.any(np.signbit(g))


def test_routed_combine_large_sampled(loom, device):
    tokens, routes, hidden = 16384, 8, 1024
    ids, weights, payload = synth.routed_inputs(tokens=tokens, routes=routes, hidden=hidden, device=device)
    g = _np(loom.routed_combine(ids, weights, payload))
    rng = np.random.default_rng(11)
    sample = np.unique(np.concatenate([[0, tokens - 1], rng.integers(0, tokens, 64)]))
    hp = payload.cpu().numpy()
    ref = oracle.routed_combine(ids.cpu().numpy()[sample], weights.cpu().numpy()[sample], hp)[0]
    assert np.array_equal(g[sample].view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ binding checks (nothing is launched)

def test_binding_rejects_short_buffers(loom, device):
    # the C ABI takes raw pointers; the binding refuses caller buffers that are
    # too small, of the wrong type or not contiguous, before anything is enqueued
    x = torch.zeros(8, 256, device=device)
    with pytest.raises(ValueError):
        loom.row_sums(x, out=torch.empty(7, device=device))
    w = torch.zeros(16, 64, dtype=torch.int32, device=device)
    v = torch.zeros(2, 64, dtype=torch.int32, device=device)
    with pytest.raises(ValueError):
        loom.i8_dequant_dot(w, torch.ones(15, device=device), v)
    with pytest.raises(ValueError):
        loom.i8_dequant_dot(w, torch.ones(16, device=device), v, torch.ones(1, device=device))
    with pytest.raises(ValueError):
        loom.i8_dequant_dot(w, torch.ones(16, device=device), v, out=torch.empty(16, 1, device=device))
    with pytest.raises(ValueError):
        loom.i8_dequant_dot(w, torch.ones(16, device=device), v, acc=torch.empty(31, dtype=torch.int32, device=device))
    with pytest.raises(TypeError):
        loom.i8_dequant_dot(w, torch.ones(16, device=device), v, out=torch.empty(16, 2, dtype=torch.float16, device=device))
    off = torch.tensor([0, 3, 8], dtype=torch.int64, device=device)
    with pytest.raises(ValueError):
        loom.segment_sums(x, off, out=torch.empty(2, 255, device=device))
    with pytest.raises(ValueError):
        loom.segment_sums(x, off, tail_counts=torch.empty(1, dtype=torch.int32, device=device))
    f = torch.zeros(4, 100, dtype=torch.int32, device=device)
    s16 = torch.zeros(4, 100, dtype=torch.int16, device=device)
    r = torch.zeros(4, 64, 4, device=device)
    with pytest.raises(ValueError):
        loom.packed_dot(f, s16, r, 4, initial=torch.zeros(99, device=device))
    with pytest.raises(ValueError):
        loom.packed_dot(f, s16, r, 4, out=torch.empty(100, 2, device=device).t())
    ids = torch.zeros(3, 2, dtype=torch.int32, device=device)
    with pytest.raises(ValueError):
        loom.routed_combine(ids, torch.zeros(3, 2, device=device), torch.zeros(6, 8, device=device),
                            out=torch.empty(3, 7, device=device))
    with pytest.raises(ValueError):
        loom.sum_guarded_rows(torch.zeros(4, 32, 4, device=device), 4, 4, 32, out=torch.empty(31, device=device))
    with pytest.raises(ValueError):
        loom.copy_f32(torch.zeros(10, device=device), out=torch.empty(9, device=device))


# ------------------------------------------------------------------ launch status

def _loaded_hip_runtime():
    """The HIP runtime this process (torch and libloom.so) uses, found among the
    mapped libraries, so the call below reaches the same runtime state."""
    import ctypes
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64.so" in line}
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths.pop())


def test_stale_hip_error_is_not_reported(loom, device):
    # An unrelated HIP call that fails first (an invalid device index) leaves
    # its error as the thread's last error; a valid call must still report
    # LOOM_OK, and the same launch on the real device must compute.
    # (no torch call between the failing call and the library's: torch would
    # itself pick up the stale error)
    import ctypes
    hip = _loaded_hip_runtime()
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    x = torch.ones(40, 300, device=device)
    out = torch.empty(40, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(100000) != 0  # hipErrorInvalidDevice, current device unchanged
    st = loom.library().loom_row_sums(ctypes.c_void_p(x.data_ptr()), 40, 300, 300, ctypes.c_void_p(out.data_ptr()),
                                      stream)
    assert st == loom.OK
    assert np.all(_np(out) == 300.0)
