"""CPU-side checks of the C ABI: the library loads, exports every declared
symbol, evaluates launch geometry, and rejects bad arguments on the host
before any device call (no GPU needed: every call here returns before the
HIP runtime is touched).

Pages: "Kernels and launch configuration" (§Workload is not workgroup count,
§Evaluate the compiled launch contract).
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from tests.golden import load as golden

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "loom.h")


@pytest.fixture(scope="module")
def loom():
    import int8_dequant_dot_amd as m
    return m


@pytest.fixture(scope="module")
def lib(loom):
    return loom.library()


FAKE = 0x10000  # a 64 KiB-aligned non-null address; never dereferenced by these tests


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(loom_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(loom):
    out = subprocess.run(["nm", "-D", "--defined-only", loom.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    names = declared_symbols()
    assert len(names) >= 9
    missing = [n for n in names if n not in exported]
    assert not missing, missing


def test_library_built_for_gfx950_only(loom, tmp_path):
    # the device code objects live in the library's .hip_fatbin bundle
    blob = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", loom.LIB_PATH, str(blob)],
                   check=True)
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob.read_bytes()))
    assert targets == {b"gfx950"}, targets


def test_status_strings(loom):
    for st in range(0, -8, -1):
        assert loom.status_string(st) and loom.status_string(st) != "unknown status"
    assert loom.status_string(-99) == "unknown status"
    assert loom.version() >= 100


# ------------------------------------------------------------------ launch configuration

def test_launch_config_page_example(loom):
    tok = loom.launch_config_lookup("copy_f32")
    for n, wg, expected in golden.launch_fill():
        cfg = loom.launch_config_invoke(tok, [n])
        assert cfg["workgroups"] == (expected, 1, 1)
        assert cfg["workgroup_size"] == (wg, 1, 1)
        assert cfg["subgroup_size"] == 64 and cfg["cluster_size"] == (1, 1, 1)
        assert cfg["workgroup_storage_bytes"] == 0


def test_launch_config_matches_oracle_geometry(loom):
    tok = loom.launch_config_lookup("copy_f32")
    for n in list(range(0, 2050)) + [2 ** 31, 2 ** 32 - 256]:
        assert loom.launch_config_invoke(tok, [n])["workgroups"][0] == oracle.fill_workgroups(n, 256)


def test_launch_config_tiles(loom):
    rs = loom.launch_config_lookup("row_sums")
    for rows in (0, 1, 7, 8, 9, 63, 64, 65, 65536, 65537):
        # short rows: one wave per 2 tiles of 8 rows
        assert loom.launch_config_invoke(rs, [rows, 256])["workgroups"][0] == -(-rows // 16)
        assert loom.launch_config_invoke(rs, [rows, 768])["workgroup_size"][0] == 64
        # long rows: a workgroup per row, one wave per 4 KiB of the row, at most 16
        cfg = loom.launch_config_invoke(rs, [rows, 4096])
        assert cfg["workgroups"][0] == rows and cfg["workgroup_size"][0] == 256
        assert cfg["workgroup_storage_bytes"] == 64  # 16 wave totals in LDS
    assert loom.launch_config_invoke(rs, [8, 1024])["workgroup_size"][0] == 64
    # narrow rows: 64 / L rows per record (4 L >= cols), 8 records per wave
    for cols, rows_per_wave in ((1, 512), (4, 512), (5, 256), (32, 64), (33, 32), (128, 16)):
        assert loom.launch_config_invoke(rs, [100000, cols])["workgroups"][0] == -(-100000 // rows_per_wave), cols
    assert loom.launch_config_invoke(rs, [100000, 129])["workgroups"][0] == -(-100000 // 16)  # tiled
    assert loom.launch_config_invoke(rs, [8, 1 << 24])["workgroup_size"][0] == 1024
    seg = loom.launch_config_lookup("segment_sums")
    assert loom.launch_config_invoke(seg, [16384, 256, 33640572])["workgroups"] == (16384, 1, 1)
    assert loom.launch_config_invoke(seg, [100, 1000, 5000])["workgroups"] == (100, 4, 1)  # a wave per 256 columns
    assert loom.launch_config_invoke(seg, [5, 0, 10**9])["workgroups"] == (5, 1, 1)  # still writes the tail counts
    # few long segments (fewer than 192 segment waves, at least 1024 rows on
    # average): P parts per segment, parts of at least 512 rows on average,
    # P * waves <= 4096.  Rows of at most 512 columns split into 16 parts or
    # more take P a multiple of 8 and run the parts in runs of 8, an 8-wave
    # workgroup per run (LDS: the run's 8 part sums of one 256-column block);
    # otherwise a wave per part.
    for segments, cols, total, parts, runs in (
            (4, 256, 4 * 2**20, 1024, 128), (3, 256, 120000, 72, 9), (3, 1000, 120000, 78, 0),
            (47, 1000, 10**7, 21, 0), (48, 1000, 10**7, 1, 0), (191, 256, 10**8, 16, 2), (192, 256, 10**8, 1, 0),
            (10, 256, 10239, 1, 0), (10, 256, 10240, 2, 0), (2, 2**20, 10**6, 1, 0), (1, 4096, 2**20, 256, 0),
            (1, 256, 15 * 512, 15, 0), (1, 256, 16 * 512, 16, 2), (1, 256, 31 * 512, 24, 3),
            (1, 512, 2**21, 2048, 256), (2, 513, 2**21, 682, 0), (1, 1, 40 * 512, 40, 5), (5, 200, 6 * 512 * 5, 6, 0)):
        blocks = -(-cols // 256)
        cfg = loom.launch_config_invoke(seg, [segments, cols, total])
        if runs:
            assert parts == 8 * runs
            assert cfg["workgroups"] == (segments * runs, blocks, 1), (segments, cols, total)
            assert cfg["workgroup_size"] == (512, 1, 1) and cfg["workgroup_storage_bytes"] == 8 * 1024
        else:
            assert cfg["workgroups"] == (segments * parts, blocks, 1), (segments, cols, total)
            assert cfg["workgroup_size"] == (64, 1, 1) and cfg["workgroup_storage_bytes"] == 0
    i8 = loom.launch_config_lookup("i8_dequant_dot")
    # one vector, always a v_dot4 GEMV: rows of 6 to 8 whole 1 KiB records,
    # and rows of more than 3 and less than 12 KiB that are a multiple of 16
    # but not of 1024 bytes, a workgroup per row with a wave per 2 records (the
    # last one partly empty; LDS: the wave totals) ...
    for k, waves in ((6144, 3), (7168, 4), (8192, 4), (3088, 2), (3328, 2), (4608, 3), (8704, 5), (11008, 6),
                     (12272, 6)):
        cfg = loom.launch_config_invoke(i8, [100, k, 1])
        assert cfg["workgroups"] == (100, 1, 1) and cfg["workgroup_size"] == (64 * waves, 1, 1), k
        assert cfg["workgroup_storage_bytes"] == 4 * waves, k
    assert loom.launch_config_invoke(i8, [16384, 8192, 1])["workgroups"][0] == 16384
    # ... other rows of whole 1 KiB records, and rows of 12 KiB or more, a wave
    # per block of about 8 KiB of rows (at least one row) ...
    for k, rows_per_wave in ((1024, 8), (2048, 4), (3072, 2), (4096, 2), (5120, 1), (9216, 1), (16384, 1),
                             (130048, 1), (12292, 1), (12804, 1), (16896, 1), (131068, 1)):
        cfg = loom.launch_config_invoke(i8, [100, k, 1])
        assert cfg["workgroups"] == (-(-100 // rows_per_wave), 1, 1) and cfg["workgroup_size"] == (64, 1, 1), k
    # ... other rows longer than 512 bytes in groups of 2 rows x 512 B pieces (k
    # a multiple of 512) or 4 rows x 256 B, whole groups of about 8 KiB a wave ...
    for k, rows_per_wave in ((516, 12), (528, 12), (768, 8), (1028, 4), (1040, 4), (1280, 4), (1536, 4),
                             (2560, 2), (3072 - 16, 4), (4092, 4), (4100, 4), (8708, 4), (12284, 4)):
        cfg = loom.launch_config_invoke(i8, [100, k, 1])
        assert cfg["workgroups"] == (-(-100 // rows_per_wave), 1, 1) and cfg["workgroup_size"] == (64, 1, 1), k
    # ... and rows of up to 512 bytes packed 64 / L to a record (16 L >= k),
    # whole records of about 8 KiB a wave, at most 64 rows
    for k, rows_per_wave in ((0, 64), (4, 64), (16, 64), (100, 64), (256, 32), (260, 30), (512, 16)):
        cfg = loom.launch_config_invoke(i8, [1000, k, 1])
        assert cfg["workgroups"] == (-(-1000 // rows_per_wave), 1, 1) and cfg["workgroup_size"] == (64, 1, 1), k
    cfg = loom.launch_config_invoke(i8, [28672, 8192, 8])
    assert cfg["workgroups"][0] == 1792
    # 4 waves split k per 16-row tile; LDS: each wave's partial sums of the
    # tile's 16 rows x 8 vectors (the segment-paired kernel stages nothing)
    assert cfg["workgroup_size"] == (256, 1, 1)
    assert cfg["workgroup_storage_bytes"] == 4 * 16 * 8 * 4
    # more than 16 vectors, four column tiles: one wave per 16-vector
    # column tile, the 16-row tiles shared evenly by one or two workgroups per
    # CU (at most 8 tiles per wave); LDS: two record slots of 256 B per row
    for rows, rt, groups in ((16384, 4, 256), (28672, 7, 256), (24575, 6, 256), (24576, 6, 256), (4096, 1, 256),
                             (4097, 2, 129), (32768, 8, 256), (32769, 5, 410), (40960, 5, 512), (57344, 7, 512),
                             (65536, 8, 512), (65537, 6, 683), (5, 1, 1)):
        cfg = loom.launch_config_invoke(i8, [rows, 8192, 64])
        assert cfg["workgroups"][0] == groups == -(-rows // (16 * rt)), rows
        assert cfg["workgroup_size"] == (256, 1, 1) and cfg["workgroup_storage_bytes"] == 2 * 16 * rt * 256, rows
    # 17-32 vectors take the same kernel and geometry (the unused column
    # tiles are zeroed)
    for batch in (17, 32, 33, 64):
        assert loom.launch_config_invoke(i8, [28672, 8192, batch]) == loom.launch_config_invoke(i8, [28672, 8192, 64])
    cfg = loom.launch_config_invoke(i8, [100, 1000, 17])
    assert cfg["workgroups"][0] == 7 and cfg["workgroup_size"] == (256, 1, 1)
    assert loom.launch_config_invoke(i8, [5, 64, 33])["workgroups"][0] == 1
    assert loom.launch_config_invoke(i8, [17, 64, 2])["workgroups"][0] == 2
    # 9-16 vectors, k a multiple of 1024 from 4096 to 8192: one 16-wave
    # workgroup per CU walks the 16-row tiles; LDS: the tile (16 rows x k
    # bytes) and the 16 waves' partial tiles
    cfg = loom.launch_config_invoke(i8, [28672, 8192, 16])
    assert cfg["workgroups"][0] == 256 and cfg["workgroup_size"] == (1024, 1, 1)
    assert cfg["workgroup_storage_bytes"] == 16 * 8192 + 16 * 1024
    assert loom.launch_config_invoke(i8, [100, 5120, 9])["workgroups"][0] == 7
    assert loom.launch_config_invoke(i8, [100, 5120, 9])["workgroup_storage_bytes"] == 16 * 5120 + 16 * 1024
    # the tile-per-workgroup kernel: about 2 KiB of every row per wave, so 1
    # wave per tile up to k = 2048, 2 at 4096, 4 from 8192, and 8 from 16384
    # when there are at least 512 tiles; LDS: (waves - 1) int32 partial tiles
    # of 1 KiB and one 16 x 256 B staging tile per wave
    for shape, ks in (([28672, 8192, 8], 4), ([100, 1000, 12], 1), ([100, 9216, 12], 4), ([15, 4096, 12], 2),
                      ([100, 3072, 16], 1), ([229376, 1024, 8], 1), ([114688, 2048, 2], 1), ([57344, 4096, 8], 2),
                      ([14336, 16384, 8], 8), ([8192, 16384, 8], 8), ([8176, 16384, 8], 4), ([7168, 32768, 2], 4),
                      ([5, 65536, 2], 4), ([100, 4, 2], 1), ([100, 0, 2], 1)):
        cfg = loom.launch_config_invoke(i8, shape)
        assert cfg["workgroups"][0] == -(-shape[0] // 16), shape
        assert cfg["workgroup_size"] == (64 * ks, 1, 1), shape
        if 7 <= shape[2] <= 8 or (shape[2] <= 8 and ks == 8):
            # the segment-paired kernel: each wave's 16 rows x 4 or 8 vector slots of int32
            assert cfg["workgroup_storage_bytes"] == ks * 16 * (8 if shape[2] > 4 else 4) * 4, shape
        else:
            assert cfg["workgroup_storage_bytes"] == (ks - 1) * 1024 + ks * 4096, shape
    t = loom.launch_config_lookup("row_sum_tiles")
    assert loom.launch_config_invoke(t, [63])["workgroups"] == (1, 1, 1)
    assert loom.launch_config_invoke(t, [63])["workgroup_size"] == (64, 1, 1)


def test_one_vector_never_takes_the_matrix_cores(loom):
    # Every row length with one vector runs a v_dot4 GEMV form: a 64-lane
    # wave per block of rows with no LDS, or a workgroup per row whose LDS holds
    # one total per wave.  The matrix-core kernels use 16-row tiles and stage
    # records or partial tiles in LDS, so neither shape can be taken for theirs.
    i8 = loom.launch_config_lookup("i8_dequant_dot")
    rows = 100
    for k in list(range(0, 40000, 4)) + [65536, 131068, 1 << 20]:
        cfg = loom.launch_config_invoke(i8, [rows, k, 1])
        size, lds = cfg["workgroup_size"][0], cfg["workgroup_storage_bytes"]
        rows_form = size == 64 and lds == 0
        wide_form = cfg["workgroups"] == (rows, 1, 1) and size % 64 == 0 and lds == 4 * (size // 64)
        assert rows_form or wide_form, (k, cfg)


def test_launch_config_errors(loom, lib):
    with pytest.raises(loom.LoomError) as e:
        loom.launch_config_lookup("no_such_kernel")
    assert e.value.status == loom.ERR_UNKNOWN_EXPORT
    tok = loom.launch_config_lookup("row_sums")
    with pytest.raises(loom.LoomError) as e:
        loom.launch_config_invoke(tok, [8])  # wrong arity
    assert e.value.status == loom.ERR_TOKEN
    with pytest.raises(loom.LoomError) as e:
        loom.launch_config_invoke(99, [8, 8])
    assert e.value.status == loom.ERR_TOKEN
    with pytest.raises(loom.LoomError) as e:
        loom.launch_config_invoke(0, [8, 8])
    assert e.value.status == loom.ERR_TOKEN
    with pytest.raises(loom.LoomError) as e:
        loom.launch_config_invoke(tok, [-1, 8])
    assert e.value.status == loom.ERR_RANGE
    with pytest.raises(loom.LoomError) as e:  # grid beyond 2^31-1 workgroups
        loom.launch_config_invoke(loom.launch_config_lookup("copy_f32"), [2 ** 31 * 256])
    assert e.value.status == loom.ERR_RANGE
    # a grid of 2^32 work-items or more is never launched (HIP refuses it):
    # one element per work-item stops at 2^32 - 256 elements ...
    copy = loom.launch_config_lookup("copy_f32")
    assert loom.launch_config_invoke(copy, [2 ** 32 - 256])["workgroups"][0] == 2 ** 24 - 1
    for n in (2 ** 32 - 255, 2 ** 32, 2 ** 33 + 5):
        with pytest.raises(loom.LoomError) as e:
            loom.launch_config_invoke(copy, [n])
        assert e.value.status == loom.ERR_RANGE
    # ... while the kernels with a unit per workgroup take every grid.x-th unit
    # past the limit (segments, long rows, tokens, long GEMV rows)
    cap64, cap256 = (2 ** 32 - 1) // 64, (2 ** 32 - 1) // 256
    seg = loom.launch_config_lookup("segment_sums")
    assert loom.launch_config_invoke(seg, [cap64, 256, 0])["workgroups"] == (cap64, 1, 1)
    assert loom.launch_config_invoke(seg, [cap64 + 1, 256, 0])["workgroups"] == (cap64, 1, 1)
    assert loom.launch_config_invoke(seg, [2 ** 31 - 2, 1000, 2**40])["workgroups"] == (cap64, 4, 1)
    rs = loom.launch_config_lookup("row_sums")
    assert loom.launch_config_invoke(rs, [2 ** 24, 4096])["workgroups"] == (cap256, 1, 1)
    assert loom.launch_config_invoke(rs, [2 ** 31 - 1, 1 << 24])["workgroups"] == ((2 ** 32 - 1) // 1024, 1, 1)
    assert loom.launch_config_invoke(rs, [2 ** 30 - 16, 768])["workgroups"] == (2 ** 26 - 1, 1, 1)
    with pytest.raises(loom.LoomError) as e:  # row tiles: 4 work-items per row
        loom.launch_config_invoke(rs, [2 ** 30 - 15, 768])
    assert e.value.status == loom.ERR_RANGE
    rt = loom.launch_config_lookup("routed_combine")
    assert loom.launch_config_invoke(rt, [2 ** 26, 8, 1024])["workgroups"] == (cap64, 1, 1)
    i8 = loom.launch_config_lookup("i8_dequant_dot")
    assert loom.launch_config_invoke(i8, [2 ** 31 - 1, 8192, 1])["workgroups"] == (cap256, 1, 1)
    with pytest.raises(loom.LoomError) as e:  # 16-row tiles of 4 waves: 16 work-items per row
        loom.launch_config_invoke(i8, [2 ** 28, 8192, 8])
    assert e.value.status == loom.ERR_RANGE
    assert loom.launch_config_invoke(i8, [2 ** 28 - 16, 8192, 8])["workgroups"] == (2 ** 24 - 1, 1, 1)
    assert lib.loom_launch_config_lookup(None, None) == loom.ERR_NULL
    assert lib.loom_launch_config_invoke(tok, None, 2, None) == loom.ERR_NULL
    assert sorted(loom.EXPORTS) == sorted(
        n for n in loom.EXPORTS if loom.launch_config_lookup(n) > 0)


# ------------------------------------------------------------------ host-side validation
# Each call below fails a documented check and must return before touching the device.

def test_copy_validation(loom, lib):
    assert lib.loom_copy_f32(FAKE, FAKE, -1, None) == loom.ERR_RANGE
    assert lib.loom_copy_f32(None, None, 0, None) == loom.OK  # nothing to do, nothing launched
    assert lib.loom_copy_f32(None, FAKE, 5, None) == loom.ERR_NULL
    assert lib.loom_copy_f32(FAKE + 2, FAKE, 5, None) == loom.ERR_ALIGN


def test_row_sum_tiles_validation(loom, lib):
    f = lib.loom_row_sum_tiles
    assert f(FAKE, 63, 64, None, FAKE, FAKE, FAKE, None) == loom.ERR_RANGE  # count > rows_alloc
    assert f(FAKE, 63, -1, None, FAKE, FAKE, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, -1, 0, None, FAKE, FAKE, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, (1 << 26) + 1, 0, None, FAKE, FAKE, FAKE, None) == loom.ERR_RANGE
    assert f(None, 63, 8, None, FAKE, FAKE, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, 63, 8, None, None, FAKE, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, 63, 8, None, FAKE, None, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, 63, 8, None, FAKE, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE + 1, 63, 8, None, FAKE, FAKE, FAKE, None) == loom.ERR_ALIGN
    assert f(FAKE, 63, 8, FAKE + 2, FAKE, FAKE, FAKE, None) == loom.ERR_ALIGN


def test_row_sums_validation(loom, lib):
    f = lib.loom_row_sums
    assert f(FAKE, -1, 4, 4, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, 4, -1, 4, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, 1 << 31, 4, 4, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, 4, 8, 7, FAKE, None) == loom.ERR_SHAPE  # stride < cols
    assert f(FAKE, 1 << 30, 4, 1 << 40, FAKE, None) == loom.ERR_RANGE  # extent overflows
    assert f(None, 0, 4, 4, None, None) == loom.OK
    assert f(None, 4, 4, 4, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, 4, 4, 4, None, None) == loom.ERR_NULL
    assert f(FAKE + 2, 4, 4, 4, FAKE, None) == loom.ERR_ALIGN
    assert f(FAKE, 4, 4, 4, FAKE + 1, None) == loom.ERR_ALIGN


def test_segment_sums_validation(loom, lib):
    f = lib.loom_segment_sums
    assert f(FAKE, 10, FAKE, -1, 4, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, 10, FAKE, 2, -1, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, 10, FAKE, 2, (1 << 20) + 1, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, -1, FAKE, 2, 4, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, (1 << 40) + 1, FAKE, 2, 4, FAKE, None, None) == loom.ERR_RANGE
    assert f(None, 0, None, 0, 4, None, None, None) == loom.OK
    assert f(FAKE, 10, None, 2, 4, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE, 10, FAKE, 2, 4, None, None, None) == loom.ERR_NULL
    assert f(None, 10, FAKE, 2, 4, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE, 10, FAKE + 4, 2, 4, FAKE, None, None) == loom.ERR_ALIGN
    assert f(FAKE, 10, FAKE, 2, 4, FAKE, FAKE + 2, None) == loom.ERR_ALIGN


def test_i8_validation(loom, lib):
    f = lib.loom_i8_dequant_dot
    assert f(FAKE, FAKE, FAKE, None, 4, 6, 1, FAKE, None, None) == loom.ERR_SHAPE  # k % 4
    assert f(FAKE, FAKE, FAKE, None, 4, 131072, 1, FAKE, None, None) == loom.ERR_RANGE  # |acc| could overflow
    assert f(FAKE, FAKE, FAKE, None, 4, -4, 1, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, None, 4, 64, 0, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, None, 4, 64, 65, FAKE, None, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, None, -1, 64, 1, FAKE, None, None) == loom.ERR_RANGE
    assert f(None, None, None, None, 0, 64, 1, None, None, None) == loom.OK
    assert f(None, FAKE, FAKE, None, 4, 64, 1, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE, None, FAKE, None, 4, 64, 1, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, None, None, 4, 64, 1, FAKE, None, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, FAKE, None, 4, 64, 1, None, None, None) == loom.ERR_NULL
    assert f(FAKE + 2, FAKE, FAKE, None, 4, 64, 1, FAKE, None, None) == loom.ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, FAKE + 1, 4, 64, 8, FAKE, None, None) == loom.ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, None, 4, 64, 8, FAKE, FAKE + 3, None) == loom.ERR_ALIGN


def test_binding_refuses_cpu_tensors(loom):
    import torch
    with pytest.raises(TypeError):
        loom.row_sums(torch.zeros(4, 4))
    with pytest.raises(TypeError):
        loom.i8_dequant_dot(torch.zeros(4, 4, dtype=torch.int32), torch.zeros(4), torch.zeros(4, dtype=torch.int32))


def test_packed_dot_validation(loom, lib):
    f = lib.loom_packed_dot
    # (fields, scales, rhs, streams, initial, records, count, outputs, out, stream)
    assert f(FAKE, FAKE, FAKE, 64, None, 128, 129, 2048, FAKE, None) == loom.ERR_RANGE  # count > records
    assert f(FAKE, FAKE, FAKE, 64, None, 128, -1, 2048, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, 0, None, 128, 8, 2048, FAKE, None) == loom.ERR_RANGE  # no streams
    assert f(FAKE, FAKE, FAKE, 64, None, 128, 8, -1, FAKE, None) == loom.ERR_RANGE
    assert f(None, None, None, 64, None, 128, 8, 0, None, None) == loom.OK
    assert f(None, FAKE, FAKE, 64, None, 128, 8, 2048, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, FAKE, 64, None, 128, 8, 2048, None, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, FAKE + 4, 64, None, 128, 8, 2048, FAKE, None) == loom.ERR_ALIGN  # rhs needs 16 B
    assert f(FAKE, FAKE + 1, FAKE, 64, None, 128, 8, 2048, FAKE, None) == loom.ERR_ALIGN
    tok = loom.launch_config_lookup("packed_dot")
    assert loom.launch_config_invoke(tok, [2048, 128, 64])["workgroups"] == (8, 1, 1)
    assert loom.launch_config_invoke(tok, [262144, 128, 64])["workgroups"] == (256, 1, 1)  # 4 outputs per lane
    assert loom.launch_config_invoke(tok, [262146, 128, 16])["workgroups"] == (257, 1, 1)
    assert loom.launch_config_invoke(tok, [262144, 128, 128])["workgroups"] == (1024, 1, 1)  # 128 streams: one
    assert loom.launch_config_invoke(tok, [2049, 0, 3])["workgroups"] == (9, 1, 1)


def test_sum_guarded_rows_validation(loom, lib):
    f = lib.loom_sum_guarded_rows
    assert f(FAKE, 63, 64, 4, 32, FAKE, None) == loom.ERR_RANGE  # count > rows_alloc
    assert f(FAKE, 63, 8, 5, 32, FAKE, None) == loom.ERR_RANGE   # at most 4 components
    assert f(FAKE, 63, 8, 4, 33, FAKE, None) == loom.ERR_RANGE   # at most 32 lanes
    assert f(FAKE, 63, 8, -1, 32, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, 63, 8, 4, 32, None, None) == loom.ERR_NULL
    assert f(None, 63, 8, 4, 32, FAKE, None) == loom.ERR_NULL
    assert f(FAKE + 4, 63, 8, 4, 32, FAKE, None) == loom.ERR_ALIGN
    tok = loom.launch_config_lookup("sum_guarded_rows")
    cfg = loom.launch_config_invoke(tok, [63])
    assert cfg["workgroups"] == (1, 1, 1) and cfg["workgroup_size"] == (32, 1, 1)


def test_routed_combine_validation(loom, lib):
    f = lib.loom_routed_combine
    # (ids, weights, payload, num_rows, tokens, routes, hidden, out, stream)
    assert f(FAKE, FAKE, FAKE, 10, -1, 8, 64, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, -1, 4, 8, 64, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, 10, 4, (1 << 20) + 1, 64, FAKE, None) == loom.ERR_RANGE
    assert f(FAKE, FAKE, FAKE, 10, 4, 8, 66, FAKE, None) == loom.ERR_SHAPE  # hidden % 4
    assert f(None, None, None, 10, 0, 8, 64, None, None) == loom.OK
    assert f(None, FAKE, FAKE, 10, 4, 8, 64, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, None, 10, 4, 8, 64, FAKE, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, FAKE, 10, 4, 8, 64, None, None) == loom.ERR_NULL
    assert f(FAKE, FAKE, FAKE + 4, 10, 4, 8, 64, FAKE, None) == loom.ERR_ALIGN
    assert f(FAKE, FAKE, FAKE, 10, 4, 8, 64, FAKE + 8, None) == loom.ERR_ALIGN
    tok = loom.launch_config_lookup("routed_combine")
    assert loom.launch_config_invoke(tok, [256, 8, 1024])["workgroups"] == (256, 1, 1)  # 1024 columns per wave
    assert loom.launch_config_invoke(tok, [256, 8, 4096])["workgroups"] == (256, 4, 1)
    assert loom.launch_config_invoke(tok, [1, 32, 1028])["workgroups"] == (1, 2, 1)


def test_header_is_plain_c_and_links(loom, tmp_path):
    # include/loom.h is usable from C99 and C++ with no HIP or torch headers, and
    # a C caller that names every declared entry point links against libloom.so
    names = declared_symbols()
    src = tmp_path / "use_loom.c"
    src.write_text("#include \"loom.h\"\ntypedef void (*entry)(void);\nint main(void) {\n"
                   "    entry table[] = {\n"
                   + "".join(f"        (entry)&{n},\n" for n in names)
                   + "    };\n    return table[0] != 0 && loom_version() > 0 ? 0 : 1;\n}\n")
    inc = os.path.dirname(HEADER)
    for compiler, std in (("gcc", "-std=c99"), ("g++", "-std=c++11")):
        exe = tmp_path / f"use_loom_{compiler}"
        lang = ["-x", "c++"] if compiler == "g++" else []
        subprocess.run([compiler, std, "-Wall", "-Werror", "-pedantic", "-I", inc, *lang, str(src), "-x", "none",
                        "-o", str(exe), loom.LIB_PATH, "-Wl,--allow-shlib-undefined"], check=True, capture_output=True)


def _kernel_metadata(lib_path, tmp_path):
    """(name, private segment bytes, VGPRs) of every gfx950 kernel in the library: the
    .hip_fatbin section holds one offload bundle per source file."""
    llvm = "/opt/rocm/llvm/bin"
    blob = tmp_path / "fatbin.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib_path, str(blob)], check=True)
    data = blob.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    kernels = []
    for i, st in enumerate(starts):
        part, co = tmp_path / f"bundle{i}.bin", tmp_path / f"bundle{i}.co"
        part.write_bytes(data[st:starts[i + 1] if i + 1 < len(starts) else len(data)])
        subprocess.run([f"{llvm}/clang-offload-bundler", "--unbundle", "--type=o",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}", f"--output={co}"],
                       check=True, capture_output=True)
        notes = subprocess.run([f"{llvm}/llvm-readelf", "--notes", str(co)], check=True, capture_output=True,
                               text=True).stdout
        for entry in notes.split(".name:")[1:]:
            name = entry.split()[0]
            priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", entry).group(1))
            vgpr = int(re.search(r"\.vgpr_count:\s+(\d+)", entry).group(1))
            kernels.append((name, priv, vgpr))
    return kernels


def test_column_kernel_shares_rows_evenly(loom):
    # more than 16 vectors: for any row count, the 16-row tiles are split into
    # workgroups of RT tiles (1 <= RT <= 8, read back from the LDS size),
    # q = ceil(tiles / 2048) workgroups per CU at most, and the last workgroup
    # still has rows
    rng = np.random.default_rng(12)
    i8 = loom.launch_config_lookup("i8_dequant_dot")
    counts = list(rng.integers(1, 2**31 - 1, 300)) + [1, 16, 17, 4095, 4096, 4097, 32768, 32769, 2**31 - 1]
    refused = 0
    for rows in map(int, counts):
        try:
            cfg = loom.launch_config_invoke(i8, [rows, 64, 64])
        except loom.LoomError as e:
            # 8 tiles per workgroup at most: 2^32 work-items or more only past 2^31 - 128 rows
            assert e.status == loom.ERR_RANGE and rows > 2**31 - 128, rows
            refused += 1
            continue
        rt = cfg["workgroup_storage_bytes"] // (2 * 16 * 256)
        assert cfg["workgroup_storage_bytes"] == rt * 2 * 16 * 256 and 1 <= rt <= 8, rows
        tiles = -(-rows // 16)
        groups = cfg["workgroups"][0]
        assert groups == -(-rows // (16 * rt)) and (groups - 1) * 16 * rt < rows, rows
        assert groups <= 256 * -(-tiles // 2048), rows
        assert groups * 256 < 2**32, rows
    assert refused <= 1


def test_column_kernel_fits_two_workgroups_per_cu(loom, tmp_path):
    # more than 16 vectors over many rows run two 4-wave workgroups per CU, which
    # needs at most 256 registers per wave (two waves per SIMD); above that
    # the second workgroup of each CU waits for the first
    kernels = [(n, v) for n, _, v in _kernel_metadata(loom.LIB_PATH, tmp_path) if "i8_mfma_cols_kernel" in n]
    assert kernels
    assert all(v <= 256 for _, v in kernels), kernels


def test_no_kernel_spills_to_scratch(loom, tmp_path):
    # register spills go to per-lane scratch memory, an order of magnitude
    # slower than the streaming loads these kernels are built around
    kernels = _kernel_metadata(loom.LIB_PATH, tmp_path)
    names = " ".join(n for n, _, _ in kernels)
    for kernel in ("row_sums_kernel", "row_sums_wide_kernel", "segment_sums_kernel", "i8_gemv_kernel",
                   "i8_mfma_kernel", "i8_mfma_seg_kernel", "i8_mfma_rows_kernel", "i8_mfma_cols_kernel", "packed_dot_kernel", "packed_dot_spaced_kernel", "sum_guarded_rows_kernel",
                   "routed_combine_kernel", "row_sum_tiles_kernel", "copy_f32_kernel"):
        assert kernel in names, kernel
    spilled = [(n, p) for n, p, _ in kernels if p != 0]
    assert not spilled, spilled
