"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test checks an oracle function against something it does not compute:
values printed on the pages (tests/golden/), closed forms derived from the
pages' inputs, exact integer arithmetic, brute force over every byte pair, or
the proven worst-case error bound of recursive float summation.  The checks
are chosen so that a plausible slip in the oracle (a dropped row, a tail row
summed or read, a wrong stride, a transposed operand, unsigned bytes, a
missing scale) fails at least one of them.

Pages: "Tune loop unrolling and pipelining" (TUNE), "Functions and structured
control flow" (CTRL), "Kernels and launch configuration" (LAUNCH).
"""
import ctypes
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from tests.golden import load as golden

U32 = 2.0 ** -24  # unit roundoff of binary32
U64 = 2.0 ** -53


def gamma(n, u=U32):
    """Higham's gamma_n = n u / (1 - n u): bound on recursive summation of n+1 terms."""
    return n * u / (1 - n * u)


def iota64x32():
    r = np.arange(64)[:, None]
    l = np.arange(32)[None, :]
    return (1 + 32 * r + l).astype(np.float32)


# ------------------------------------------------------------------ tile split
# TUNE §Derive full tiles from a ragged loop

def test_tile_split_closed_form():
    for tile in (1, 3, 8, 16):
        for c in range(0, 4097):
            assert oracle.tile_split(c, tile) == (tile * (c // tile), c % tile), (c, tile)


def test_tile_split_boundaries():
    assert oracle.tile_split(0) == (0, 0)
    assert oracle.tile_split(7) == (0, 7)
    assert oracle.tile_split(8) == (8, 0)
    assert oracle.tile_split(63) == (56, 7)


# ------------------------------------------------------------------ launch geometry
# LAUNCH §Workload is not workgroup count

def test_fill_workgroups_page_value():
    for n, wg, expected in golden.launch_fill():
        assert oracle.fill_workgroups(n, wg) == expected


def test_fill_workgroups_cover_exactly():
    assert oracle.fill_workgroups(0) == 0
    for n in range(1, 4097):
        g = oracle.fill_workgroups(n)
        assert (g - 1) * 256 < n <= g * 256, n


def test_copy_touches_only_in_bounds():
    x = synth.copy_inputs().numpy()
    out = np.full(1024, -1.0, np.float32)
    oracle.lib().oracle_copy_f32(x.ctypes.data, out.ctypes.data, x.size)
    assert np.array_equal(out[:1009].view(np.uint32), x.view(np.uint32))
    assert np.all(out[1009:] == -1.0)


# ------------------------------------------------------------------ tiled row sum
# TUNE §Derive full tiles (@guide.sum_full_tiles)

def test_row_sum_tiles_iota_closed_form():
    # row r of the iota tile sums to sum_l (1 + 32 r + l) = 528 + 1024 r, so the
    # full tiles up to F contribute 528 F + 512 F (F - 1); all partial sums are
    # integers below 2**24, hence exact in any order.
    v = iota64x32()[:63]
    for count in range(64):
        F = 8 * (count // 8)
        sums, fr, tc = oracle.row_sum_tiles(v, count)
        assert (fr, tc) == (F, count % 8)
        assert np.all(sums == 528 * F + 512 * F * (F - 1)), count


def test_row_sum_tiles_derived_values():
    v = iota64x32()[:63]
    assert oracle.row_sum_tiles(v, 8)[0][0] == 32896
    assert oracle.row_sum_tiles(v, 16)[0][0] == 131328
    assert oracle.row_sum_tiles(v, 63)[0][0] == 1606528
    assert oracle.row_sum_tiles(v, 7)[0][0] == 0  # tail only: nothing summed


def test_row_sum_tiles_initial_per_lane():
    v = iota64x32()[:63]
    init = np.arange(32, dtype=np.float32) * 3 - 40
    for count in (0, 9, 63):
        F = 8 * (count // 8)
        sums, _, _ = oracle.row_sum_tiles(v, count, init)
        assert np.array_equal(sums, init + np.float32(528 * F + 512 * F * (F - 1)))


def test_row_sum_tiles_never_reads_tail():
    rng = np.random.default_rng(0)
    for count in range(64):
        F = 8 * (count // 8)
        v = rng.integers(-8, 9, size=(63, 32)).astype(np.float32)
        poisoned = v.copy()
        poisoned[F:] = np.nan
        a = oracle.row_sum_tiles(v, count)[0]
        b = oracle.row_sum_tiles(poisoned, count)[0]
        assert np.array_equal(a, b)
        # integer data: exact, independent of order
        assert np.all(a == v[:F].astype(np.int64).sum())


def test_row_sum_tiles_random_within_bound():
    values, count = synth.tile_inputs()
    v = values.numpy()
    F = 8 * (count // 8)
    sums = oracle.row_sum_tiles(v, count)[0]
    exact = math.fsum(float(t) for t in v[:F].ravel())
    absum = math.fsum(abs(float(t)) for t in v[:F].ravel())
    # 32 adds per row plus one carried add per row: at most F*32 roundings.
    assert abs(float(sums[0]) - exact) <= gamma(F * 32) * absum + 1e-30


# ------------------------------------------------------------------ row sums

def test_row_sums_integer_exact():
    for rows in range(0, 18):
        for cols in (1, 5, 33, 256):
            r = np.arange(rows)[:, None]
            c = np.arange(cols)[None, :]
            x = (((r + 3 * c) % 7) - 3).astype(np.float32)
            out, d, a = oracle.row_sums(x)
            assert np.array_equal(out, x.astype(np.int64).sum(1).astype(np.float32))
            assert np.array_equal(a, np.abs(x).astype(np.int64).sum(1).astype(np.float64))


def test_row_sums_strided():
    rng = np.random.default_rng(1)
    rows, cols, stride = 11, 37, 44
    x = rng.integers(-5, 6, size=(rows, stride)).astype(np.float32)
    x[:, cols:] = np.nan  # padding between rows must never be read
    out = np.empty(rows, np.float32)
    oracle.lib().oracle_row_sums(x.ctypes.data, rows, cols, stride, out.ctypes.data, None, None)
    assert np.array_equal(out, x[:, :cols].astype(np.int64).sum(1).astype(np.float32))


def test_row_sums_random_within_bound():
    x = synth.dense_rows(synth.DENSE.seed, 0, 19, 4096).numpy()
    out, d, a = oracle.row_sums(x)
    for i in range(x.shape[0]):
        exact = math.fsum(float(t) for t in x[i])
        absum = math.fsum(abs(float(t)) for t in x[i])
        assert abs(float(out[i]) - exact) <= gamma(x.shape[1] - 1) * absum
        assert abs(d[i] - exact) <= gamma(x.shape[1] - 1, U64) * absum
        assert abs(a[i] - absum) <= gamma(x.shape[1] - 1, U64) * absum


# ------------------------------------------------------------------ segment sums
# TUNE §Keep one checked source / §Complete correctness cases (the printed vectors)

def test_segment_sums_page_vectors():
    v = iota64x32()
    lanes = np.arange(32)
    for case, count, offset, step in golden.sum_rows_iota():
        out, tails, _, _ = oracle.segment_sums(v, np.array([0, count]))
        assert np.array_equal(out[0], (offset + step * lanes).astype(np.float32)), case
        assert tails[0] == count % 8


def test_segment_sums_page_closed_form():
    # the page's exact answer for N rows: N (lane + 1) + 16 N (N - 1)
    v = iota64x32()
    lanes = np.arange(32)
    for n in range(65):
        out = oracle.segment_sums(v, np.array([0, n]))[0][0]
        assert np.array_equal(out, (n * (lanes + 1) + 16 * n * (n - 1)).astype(np.float32)), n


def test_segment_sums_empty_is_positive_zero():
    v = np.full((4, 8), -3.0, np.float32)
    out, tails, _, _ = oracle.segment_sums(v, np.array([0, 0, 4, 4]))
    assert np.all(out[0] == 0) and not np.any(np.signbit(out[0]))
    assert not np.any(np.signbit(out[2]))
    assert np.all(out[1] == -12.0)
    assert list(tails) == [0, 4, 0]


def test_segment_sums_integer_exact_ragged():
    rng = np.random.default_rng(2)
    lengths = np.array([0, 1, 7, 8, 9, 15, 16, 17, 0, 3, 64, 5])
    off = np.concatenate([[0], np.cumsum(lengths)])
    cols = 13
    x = rng.integers(-9, 10, size=(off[-1], cols)).astype(np.float32)
    out, tails, d, a = oracle.segment_sums(x, off)
    for s in range(lengths.size):
        ref = x[off[s]:off[s + 1]].astype(np.int64).sum(0)
        assert np.array_equal(out[s], ref.astype(np.float32)), s
        assert tails[s] == lengths[s] % 8


def test_segment_sums_random_within_bound():
    lengths = synth.segment_lengths(synth.SEGMENTS.seed, 6, 300)
    off = synth.segment_offsets(lengths)
    x = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), 256).numpy()
    out, tails, d, a = oracle.segment_sums(x, off.numpy())
    for s in range(6):
        blk = x[int(off[s]):int(off[s + 1])]
        n = blk.shape[0]
        for c in (0, 1, 100, 255):
            exact = math.fsum(float(t) for t in blk[:, c])
            absum = math.fsum(abs(float(t)) for t in blk[:, c])
            assert abs(float(out[s, c]) - exact) <= gamma(max(n - 1, 0)) * absum


# ------------------------------------------------------------------ int8 dequant dot
# TUNE §Apply the same controls to a packed dot product

def test_i8_acc_matches_exact_int_matmul():
    rng = np.random.default_rng(3)
    for rows, k, batch in [(5, 4, 1), (17, 36, 3), (33, 1028, 8), (3, 8192, 2)]:
        w = rng.integers(-128, 128, size=(rows, k), dtype=np.int64)
        x = rng.integers(-128, 128, size=(batch, k), dtype=np.int64)
        ws = np.ones(rows, np.float32)
        _, acc = oracle.i8_dequant_dot(w.astype(np.int8), ws, x.astype(np.int8))
        assert np.array_equal(acc, (w @ x.T).astype(np.int32))


def _pack(bytes_2d):
    """Pack int8 elements into little-endian int32 words with explicit shifts."""
    b = np.asarray(bytes_2d, np.int64) & 0xFF
    n, k = b.shape
    words = np.zeros((n, k // 4), np.int64)
    for j in range(4):
        words |= b[:, j::4] << (8 * j)
    words = np.where(words >= 1 << 31, words - (1 << 32), words)
    return words.astype(np.int32)


def test_i8_all_byte_pairs_each_position():
    # every signed byte value times every other, at each byte position of a
    # packed word: pins sign extension and the element order within a word.
    a = np.arange(-128, 128)
    for pos in range(4):
        wb = np.zeros((256, 4), np.int64)
        wb[:, pos] = a
        xb = np.zeros((256, 4), np.int64)
        xb[:, pos] = a
        w = _pack(wb).view(np.int8)  # byte view of the packed words
        x = _pack(xb).view(np.int8)
        _, acc = oracle.i8_dequant_dot(w, np.ones(256, np.float32), x)
        assert np.array_equal(acc, np.outer(a, a).astype(np.int32)), pos


def test_i8_extremes_and_overflow_limit():
    for k in (4, 8192, 131068):
        w = np.full((1, k), -128, np.int8)
        x = np.full((2, k), -128, np.int8)
        x[1] = 127
        _, acc = oracle.i8_dequant_dot(w, np.ones(1, np.float32), x)
        assert acc[0, 0] == 16384 * k and acc[0, 1] == -16256 * k
    with pytest.raises(OverflowError):
        oracle.i8_dequant_dot(np.full((1, 131072), -128, np.int8), np.ones(1, np.float32),
                              np.full((1, 131072), -128, np.int8))


def test_i8_one_hot_selects_weight_column():
    rng = np.random.default_rng(4)
    rows, k, batch = 9, 64, 5
    w = rng.integers(-128, 128, size=(rows, k)).astype(np.int8)
    cols = [0, 5, 17, 40, 63]
    x = np.zeros((batch, k), np.int8)
    for b, c in enumerate(cols):
        x[b, c] = 1
    _, acc = oracle.i8_dequant_dot(w, np.ones(rows, np.float32), x)
    assert np.array_equal(acc, w[:, cols].astype(np.int32))


def test_i8_scale_epilogue():
    rng = np.random.default_rng(5)
    rows, k, batch = 64, 256, 8
    w = rng.integers(-128, 128, size=(rows, k)).astype(np.int8)
    x = rng.integers(-128, 128, size=(batch, k)).astype(np.int8)
    # unit scales: the output is the accumulator itself (|acc| < 2**24, exact)
    out, acc = oracle.i8_dequant_dot(w, np.ones(rows, np.float32), x, np.ones(batch, np.float32))
    assert np.array_equal(out, acc.astype(np.float32))
    # power-of-two scales: products are exact
    ws = (2.0 ** rng.integers(-12, 3, size=rows)).astype(np.float32)
    xs = (2.0 ** rng.integers(-6, 6, size=batch)).astype(np.float32)
    out, acc = oracle.i8_dequant_dot(w, ws, x, xs)
    assert np.array_equal(out.astype(np.float64), acc * ws[:, None].astype(np.float64) * xs[None, :])
    # general scales: three roundings (int->f32 and two products) of the exact value
    ws = synth.scales(9, synth.S_WSCALE, 0, rows).numpy()
    xs = synth.scales(9, synth.S_XSCALE, 0, batch).numpy()
    out, acc = oracle.i8_dequant_dot(w, ws, x, xs)
    bound = 3 * U32 + 3 * U32 * U32
    for r in range(rows):
        for b in range(batch):
            exact = Fraction(int(acc[r, b])) * Fraction(float(ws[r])) * Fraction(float(xs[b]))
            assert abs(Fraction(float(out[r, b])) - exact) <= bound * abs(exact)
    # without x_scale the second product is skipped
    out1, _ = oracle.i8_dequant_dot(w, ws, x)
    out2, _ = oracle.i8_dequant_dot(w, ws, x, np.ones(batch, np.float32))
    assert np.array_equal(out1, out2)


def test_i8_large_acc_conversion_rounds_to_nearest():
    # |acc| > 2**24: int -> f32 rounds; check against exact rounding via Fraction
    k = 2048
    w = np.full((1, k), -128, np.int8)
    x = np.full((1, k), -127, np.int8)
    x[0, 0] = -125
    out, acc = oracle.i8_dequant_dot(w, np.ones(1, np.float32), x)
    exact = 128 * 127 * k - 256
    assert acc[0, 0] == exact
    assert float(out[0, 0]) == float(np.float32(exact))  # numpy's int->f32 is RNE
    assert abs(float(out[0, 0]) - exact) <= 2.0 ** (math.floor(math.log2(exact)) - 24)


# ------------------------------------------------------------------ generator pins

def test_generator_is_published_splitmix64():
    d = synth.draws(11, 2, 5, 64)
    key = synth.stream_key(11, 2)
    ref = [synth.splitmix64_scalar(key + (i + 1) * 0x9E3779B97F4A7C15) for i in range(5, 69)]
    assert [v & ((1 << 64) - 1) for v in d.tolist()] == ref
    # known first output of the SplitMix64 reference with state 0 (Vigna's splitmix64.c)
    assert synth.splitmix64_scalar(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF


def test_generator_subranges_consistent():
    a = synth.normal(4, 0, 0, 1000)
    b = synth.normal(4, 0, 300, 200)
    assert np.array_equal(a[300:500].numpy(), b.numpy())
    c = synth.int8_uniform(5, synth.S_W, 0, 1000)
    e = synth.int8_uniform(5, synth.S_W, 13, 501)
    assert np.array_equal(c[13:514].numpy(), e.numpy())


def test_generator_distributions():
    x = synth.normal(1, 0, 0, 200000).numpy()
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.02 and np.abs(x).max() <= 6
    u = synth.uniform_pm1(1, 0, 0, 200000).numpy()
    assert u.min() >= -1 and u.max() < 1 and abs(u.mean()) < 0.01
    s = synth.scales(1, 5, 0, 10000).numpy()
    assert s.min() >= 1e-3 and s.max() <= 1e-2
    L = synth.segment_lengths(1, 20000, 4096).numpy()
    assert L.min() == 0 and L.max() == 4096


# ------------------------------------------------------------------ packed dot (pages' literal form)
# TUNE §Apply the same controls to a packed dot product

def test_f16_decoder_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32).view(np.uint32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32).view(np.uint32)
    nan = np.isnan(bits.view(np.float16))
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(got[nan].view(np.float32)))


def _packed(records, outputs, streams, seed=0):
    rng = np.random.default_rng(seed)
    fields = rng.integers(-2 ** 31, 2 ** 31, size=(records, outputs), dtype=np.int64).astype(np.int32)
    scales = rng.uniform(1e-3, 1e-2, size=(records, outputs)).astype(np.float16).view(np.uint16)
    rhs = rng.standard_normal((records, streams, 4)).astype(np.float32)
    return fields, scales, rhs


def test_packed_dot_empty_is_initial():
    fields, scales, rhs = _packed(4, 70, 64)
    init = np.linspace(-3, 3, 70).astype(np.float32)
    assert np.array_equal(oracle.packed_dot(fields, scales, rhs, 0, init)[0], init)
    assert np.array_equal(oracle.packed_dot(fields, scales, rhs, 0)[0], np.zeros(70, np.float32))


def test_packed_dot_one_hot_selects_signed_bytes():
    # unit scales and a one-hot activation pick byte j of every record: an exact
    # integer sum that pins sign extension and the byte order of the word
    records, outputs, streams = 9, 130, 64
    fields, _, _ = _packed(records, outputs, streams, 1)
    ones = np.full((records, outputs), 0x3C00, np.uint16)  # binary16 1.0
    b = fields.view(np.uint8).reshape(records, outputs, 4).view(np.int8).astype(np.int64)
    for j in range(4):
        rhs = np.zeros((records, streams, 4), np.float32)
        rhs[:, :, j] = 1.0
        out = oracle.packed_dot(fields, ones, rhs, records)[0]
        assert np.array_equal(out, b[:, :, j].sum(0).astype(np.float32)), j


def test_packed_dot_stream_mapping_and_scale():
    # every byte 1 in position 0, scale 2^-3, stream s carries activation s+1:
    # output o accumulates count * 2^-3 * (o mod 64 + 1)
    records, outputs, streams, count = 5, 200, 64, 4
    fields = np.full((records, outputs), 1, np.int32)
    scales = np.full((records, outputs), 0x3000, np.uint16)  # binary16 0.125
    rhs = np.zeros((records, streams, 4), np.float32)
    rhs[:, :, 0] = (np.arange(streams) + 1)[None, :]
    out = oracle.packed_dot(fields, scales, rhs, count)[0]
    assert np.array_equal(out, (count * 0.125 * (np.arange(outputs) % 64 + 1)).astype(np.float32))


def test_packed_dot_serial_accumulation_order():
    # the reading: each product is added to the carried sum in turn.  Starting
    # at 2^24 with four products of 1.0, a serial f32 recurrence stays at 2^24
    # (each +1 rounds away), while summing the products first would give 2^24+4.
    fields = np.array([[0x01010101]], np.int32)
    scales = np.array([[0x3C00]], np.uint16)
    rhs = np.ones((1, 1, 4), np.float32)
    out = oracle.packed_dot(fields, scales, rhs, 1, np.array([2.0 ** 24], np.float32))[0]
    assert out[0] == np.float32(2.0 ** 24)


def test_packed_dot_random_within_bound():
    records, outputs, streams = 14, 40, 64
    fields, scales, rhs = _packed(records, outputs, streams, 2)
    init = np.random.default_rng(3).standard_normal(outputs).astype(np.float32)
    out, d, a = oracle.packed_dot(fields, scales, rhs, records, init)
    b = fields.view(np.uint8).reshape(records, outputs, 4).view(np.int8)
    sc = scales.view(np.float16).astype(np.float64)
    n = 4 * records
    for o in range(outputs):
        exact = Fraction(float(init[o]))
        absum = abs(float(init[o]))
        for r in range(records):
            for j in range(4):
                t = Fraction(int(b[r, o, j])) * Fraction(float(sc[r, o])) * Fraction(float(rhs[r, o % 64, j]))
                exact += t
                absum += abs(float(t))
        # byte * scale is exact in f32 (8 x 11 significant bits); each product
        # with the activation rounds once, then n recursive additions
        assert abs(Fraction(float(out[o])) - exact) <= gamma(n + 1) * absum
        assert abs(d[o] - float(exact)) <= gamma(n + 1, U64) * absum + 1e-300


# ------------------------------------------------------------------ guarded ragged rows
# TUNE §Keep guards and inner loops in the source (@guide.sum_guarded_rows)

def _guarded_iota():
    r = np.arange(63)[:, None, None]
    l = np.arange(32)[None, :, None]
    c = np.arange(4)[None, None, :]
    return (1 + 4 * (32 * r + l) + c).astype(np.float32)


def test_guarded_rows_closed_form():
    # active lane l, N rows, C components: sum_r sum_c (1 + 128 r + 4 l + c)
    #   = N C (1 + 4 l) + 64 C N (N - 1) + N C (C - 1) / 2; inactive lanes give 0
    v = _guarded_iota()
    lanes = np.arange(32)
    for n in (0, 1, 2, 3, 4, 5, 8, 62, 63):
        for cols in range(5):
            for active in (0, 1, 17, 32):
                out = oracle.sum_guarded_rows(v, n, cols, active)
                want = n * cols * (1 + 4 * lanes) + 64 * cols * n * (n - 1) + n * cols * (cols - 1) // 2
                want = np.where(lanes < active, want, 0).astype(np.float32)
                assert np.array_equal(out, want), (n, cols, active)


def test_guarded_rows_never_read_outside_guards():
    rng = np.random.default_rng(6)
    for n, cols, active in [(63, 4, 32), (5, 2, 17), (4, 3, 1), (1, 1, 31), (62, 4, 0)]:
        v = rng.integers(-9, 10, size=(63, 32, 4)).astype(np.float32)
        poisoned = v.copy()
        poisoned[n:] = np.nan            # rows at or beyond count (the padded row is not even allocated)
        poisoned[:, active:] = np.nan    # inactive lanes
        poisoned[:, :, cols:] = np.nan   # components beyond the inner extent
        a = oracle.sum_guarded_rows(v, n, cols, active)
        b = oracle.sum_guarded_rows(poisoned, n, cols, active)
        assert np.array_equal(a, b) and not np.any(np.isnan(b))
        exact = v[:n, :, :cols].astype(np.int64).sum((0, 2))
        assert np.array_equal(b, np.where(np.arange(32) < active, exact, 0).astype(np.float32))


def test_guarded_rows_random_within_bound():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((63, 32, 4)).astype(np.float32)
    out = oracle.sum_guarded_rows(v, 63, 4, 32)
    for lane in range(32):
        terms = [float(t) for t in v[:, lane, :].ravel()]
        assert abs(float(out[lane]) - math.fsum(terms)) <= gamma(len(terms) + 16) * math.fsum(abs(t) for t in terms)


# ------------------------------------------------------------------ routed row combine
# TUNE §Separate route and payload lookahead

def test_routed_combine_missing_routes_read_nothing():
    rng = np.random.default_rng(8)
    tokens, routes, num_rows, hidden = 7, 8, 20, 12
    payload = rng.integers(-5, 6, size=(num_rows, hidden)).astype(np.float32)
    ids = rng.integers(0, num_rows, size=(tokens, routes)).astype(np.int32)
    weights = rng.integers(-3, 4, size=(tokens, routes)).astype(np.float32)
    missing = rng.random((tokens, routes)) < 0.4
    ids[missing] = np.where(rng.random(missing.sum()) < 0.5, -1 - rng.integers(0, 5, missing.sum()),
                            num_rows + rng.integers(0, 5, missing.sum()))
    ids[0, 0], ids[0, 1] = -(2 ** 31), num_rows   # extremes of both sides
    missing[0, :2] = True
    weights[missing] = np.nan                      # must never be read
    out = oracle.routed_combine(ids, weights, payload)[0]
    # exact integer reference over the valid routes
    ref = np.zeros((tokens, hidden), np.int64)
    for t in range(tokens):
        for i in range(routes):
            if not missing[t, i]:
                ref[t] += int(weights[t, i]) * payload[ids[t, i]].astype(np.int64)
    assert np.array_equal(out, ref.astype(np.float32))


def test_routed_combine_single_route_copies_row():
    rng = np.random.default_rng(9)
    payload = rng.standard_normal((30, 17)).astype(np.float32)
    ids = np.full((5, 4), -1, np.int32)
    weights = np.zeros((5, 4), np.float32)
    for t in range(5):
        ids[t, t % 4] = 3 * t + 1
        weights[t, t % 4] = 1.0
    out = oracle.routed_combine(ids, weights, payload)[0]
    assert np.array_equal(out, payload[[1, 4, 7, 10, 13]])
    assert np.all(oracle.routed_combine(np.full((2, 3), -7, np.int32), np.ones((2, 3), np.float32), payload)[0] == 0)


def test_routed_combine_duplicates_and_order():
    # the same row twice contributes twice; routes are added in order, one at a
    # time: 2^24 followed by two 1's stays 2^24 in f32
    payload = np.array([[2.0 ** 24], [1.0]], np.float32)
    out = oracle.routed_combine(np.array([[0, 1, 1]], np.int32), np.ones((1, 3), np.float32), payload)[0]
    assert out[0, 0] == np.float32(2.0 ** 24)
    out = oracle.routed_combine(np.array([[1, 1, 1]], np.int32), np.array([[2, 3, 4]], np.float32), payload)[0]
    assert out[0, 0] == 9.0


def test_routed_combine_random_within_bound():
    rng = np.random.default_rng(10)
    tokens, routes, num_rows, hidden = 6, 32, 64, 9
    payload = rng.standard_normal((num_rows, hidden)).astype(np.float32)
    ids = rng.integers(-4, num_rows + 4, size=(tokens, routes)).astype(np.int32)
    weights = rng.random((tokens, routes)).astype(np.float32)
    out, d, a = oracle.routed_combine(ids, weights, payload)
    for t in range(tokens):
        valid = [i for i in range(routes) if 0 <= ids[t, i] < num_rows]
        for c in range(hidden):
            terms = [Fraction(float(weights[t, i])) * Fraction(float(payload[ids[t, i], c])) for i in valid]
            exact = sum(terms, Fraction(0))
            absum = float(sum(abs(x) for x in terms))
            assert abs(Fraction(float(out[t, c])) - exact) <= gamma(len(valid) + 1) * absum
