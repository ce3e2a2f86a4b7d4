"""Seeded, counter-based synthetic inputs for the streaming-reduction workloads.

This module is shared by the oracle tests, the GPU parity tests and the benchmark.
It holds no arithmetic of the method itself (no sums, no dot products, no tiling):
only random draws and the shapes of the workloads.

Generator
---------
Every value is a pure function of ``(seed, stream, index)``: draw ``i`` of a stream
is the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) applied to the Weyl state
``key + (i + 1) * 0x9E3779B97F4A7C15``, where ``key`` is itself a SplitMix64 draw
of ``seed`` and ``stream``.  Because draws are addressed by index, any subset of a
large input (a sampled row, one segment) can be regenerated on its own, on the
CPU or on the GPU, with identical bits.

All arithmetic is 64-bit integer (wrapping), followed by conversions that are
exact in float32, or by a single float64 multiply-add rounded once to float32.
Both are correctly rounded IEEE operations, so a tensor generated on ``cuda:0``
is bit-identical to the same tensor generated on the CPU.

Distributions
-------------
* ``uniform_pm1``: float32 ``(u24 - 2**23) * 2**-23`` -- uniform on [-1, 1) with
  24-bit resolution, exact in float32.
* ``normal``: Irwin-Hall approximation of N(0, 1): the sum of twelve 16-bit
  uniforms minus their mean, scaled by 2**-16.  Mean 0, variance 1, support
  [-6, 6]; every value is exact in float32.
* ``int8_uniform``: independent bytes, uniform over [-128, 127].
* ``uniform_range``: float32 rounding of ``lo + u53 * (hi - lo)`` computed in float64.
* ``randint``: ``lo + (draw >> 1) mod (hi - lo + 1)``.
"""
from __future__ import annotations

import dataclasses

import torch

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(u: int) -> int:
    """Unsigned 64-bit constant as the int64 with the same bits."""
    u &= (1 << 64) - 1
    return u - (1 << 64) if u >= (1 << 63) else u


def _lshr(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bits (torch's >> is arithmetic)."""
    if k == 0:
        return x
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output function on int64 tensors (wrapping arithmetic)."""
    z = (z ^ _lshr(z, 30)) * _s64(_M1)
    z = (z ^ _lshr(z, 27)) * _s64(_M2)
    return z ^ _lshr(z, 31)


def splitmix64_scalar(state: int) -> int:
    """Reference SplitMix64 output function on one Python int (for pinning the tensor form)."""
    mask = (1 << 64) - 1
    z = state & mask
    z = ((z ^ (z >> 30)) * _M1) & mask
    z = ((z ^ (z >> 27)) * _M2) & mask
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    """Per-stream key: one SplitMix64 draw of (seed, stream)."""
    return splitmix64_scalar((seed * 0x100000001B3 + stream * _GAMMA + 0x632BE59BD9B4E019))


def draws(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Draws ``start .. start+count-1`` of stream ``(seed, stream)`` as int64 bit patterns."""
    key = _s64(stream_key(seed, stream))
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix(idx * _s64(_GAMMA) + key)


# ---------------------------------------------------------------- distributions

def uniform_pm1(seed, stream, start, count, device="cpu") -> torch.Tensor:
    """float32 uniform on [-1, 1) with 2**-23 resolution (exact conversion)."""
    u24 = _lshr(draws(seed, stream, start, count, device), 40)
    return (u24 - (1 << 23)).to(torch.float32) * (2.0 ** -23)


def normal(seed, stream, start, count, device="cpu") -> torch.Tensor:
    """float32 Irwin-Hall(12) approximation of N(0,1); three draws per value."""
    z = draws(seed, stream, 3 * start, 3 * count, device).view(count, 3)
    s = torch.zeros(count, dtype=torch.int64, device=device)
    for field in range(4):
        s += (_lshr(z, 16 * field) & 0xFFFF).sum(dim=1)
    # E[s] = 12 * 32767.5 = 393210; |s - 393210| < 2**19, exact in float32.
    return (s - 393210).to(torch.float32) * (2.0 ** -16)


def int8_uniform(seed, stream, start, count, device="cpu") -> torch.Tensor:
    """int8 uniform over [-128, 127]; byte j of draw i is element 8*i + j."""
    first = start // 8
    last = (start + count + 7) // 8
    z = draws(seed, stream, first, last - first, device)
    b = z.contiguous().view(torch.uint8).view(torch.int8)  # little-endian bytes
    off = start - 8 * first
    return b[off:off + count]


def uniform_range(seed, stream, start, count, lo, hi, device="cpu") -> torch.Tensor:
    """float32 rounding of lo + u * (hi - lo), u uniform on [0, 1) with 53 bits, in float64."""
    u = _lshr(draws(seed, stream, start, count, device), 11).to(torch.float64) * (2.0 ** -53)
    return (lo + u * (hi - lo)).to(torch.float32)


def randint(seed, stream, start, count, lo, hi, device="cpu") -> torch.Tensor:
    """int64 in [lo, hi] (inclusive)."""
    z = _lshr(draws(seed, stream, start, count, device), 1)
    return lo + torch.remainder(z, hi - lo + 1)


def fill_chunked(out: torch.Tensor, fn, seed, stream, chunk=1 << 26, **kw) -> torch.Tensor:
    """Fill a contiguous tensor with ``fn`` in index chunks (bounded temporaries)."""
    flat = out.view(-1)
    n = flat.numel()
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        flat[a:b] = fn(seed, stream, a, b - a, device=out.device, **kw)
    return out


# ---------------------------------------------------------------- workloads
# Streams: each input of each workload has its own stream id, so sub-ranges
# (rows, segments) can be regenerated independently.

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    desc: str


TILE = Workload("tile_63x32", 1, "one 63x32 f32 tile, N(0,1), count uniform in [0,63]")
COPY = Workload("copy_1009", 2, "1009-element f32 copy, N(0,1), workgroup size 256")
DENSE = Workload("row_sum_65536x4096", 3, "dense row sum 65536x4096 f32, uniform[-1,1]")
SEGMENTS = Workload("segment_sums_16384x256", 4, "16384 segments, lengths U{0..4096}, 256 f32 cols N(0,1)")
GEMV = Workload("i8_dot_16384x8192", 5, "int8 16384x8192 weights, per-row scale, one int8 vector")
BATCHED = Workload("i8_dot_28672x8192x8", 6, "int8 28672x8192 weights x 8 int8 vectors, row and vector scales")
PACKED = Workload("packed_dot_2048x128", 7, "2048 outputs x 128 records: packed s8 words, f16 scales, 64 f32 streams")
ROUTED = Workload("routed_combine", 8, "tokens x routes of (row id, weight) over expert-output rows of 1024 f32")

# stream ids
S_VALUES, S_COUNT, S_INITIAL, S_LENGTHS, S_W, S_WSCALE, S_X, S_XSCALE = range(8)


def tile_inputs(seed=TILE.seed, rows=63, device="cpu"):
    """values [rows][32] N(0,1) and count uniform in [0, rows]."""
    values = normal(seed, S_VALUES, 0, rows * 32, device).view(rows, 32)
    count = int(randint(seed, S_COUNT, 0, 1, 0, rows)[0])
    return values, count


def copy_inputs(seed=COPY.seed, n=1009, device="cpu"):
    return normal(seed, S_VALUES, 0, n, device)


def dense_rows(seed, row_start, row_count, cols, device="cpu"):
    """Rows [row_start, row_start+row_count) of a dense uniform[-1,1) matrix with ``cols`` columns."""
    return uniform_pm1(seed, S_VALUES, row_start * cols, row_count * cols, device).view(row_count, cols)


def dense_matrix(seed, rows, cols, device="cpu"):
    out = torch.empty(rows, cols, dtype=torch.float32, device=device)
    return fill_chunked(out, uniform_pm1, seed, S_VALUES)


def segment_lengths(seed, segments, max_len, device="cpu"):
    return randint(seed, S_LENGTHS, 0, segments, 0, max_len, device)


def segment_offsets(lengths: torch.Tensor) -> torch.Tensor:
    """CSR offsets [segments+1] from lengths (prefix sum; input layout, not the method)."""
    off = torch.zeros(lengths.numel() + 1, dtype=torch.int64, device=lengths.device)
    off[1:] = torch.cumsum(lengths, 0)
    return off


def segment_rows(seed, row_start, row_count, cols, device="cpu"):
    return normal(seed, S_VALUES, row_start * cols, row_count * cols, device).view(row_count, cols)


def segment_matrix(seed, total_rows, cols, device="cpu"):
    out = torch.empty(total_rows, cols, dtype=torch.float32, device=device)
    return fill_chunked(out, normal, seed, S_VALUES)


def i8_rows(seed, stream, row_start, row_count, k, device="cpu"):
    """Rows of an int8 matrix with k columns, uniform over [-128, 127]."""
    return int8_uniform(seed, stream, row_start * k, row_count * k, device).view(row_count, k)


def i8_matrix(seed, stream, rows, k, device="cpu"):
    out = torch.empty(rows, k, dtype=torch.int8, device=device)
    return fill_chunked(out, int8_uniform, seed, stream)


def scales(seed, stream, start, count, device="cpu"):
    """Per-row or per-vector scales uniform in [1e-3, 1e-2]."""
    return uniform_range(seed, stream, start, count, 1e-3, 1e-2, device)


def f16_scales(seed, stream, start, count, device="cpu") -> torch.Tensor:
    """binary16 bit patterns (as int16) of positive scales 2**e * (1 + m/1024),
    e uniform in {-10..-7}, m uniform in [0, 1024): values in [2**-10, 2**-6).
    Built from integer draws only, so CPU and GPU give identical bits."""
    z = _lshr(draws(seed, stream, start, count, device), 1)
    e = torch.remainder(z, 4) - 10
    m = torch.remainder(_lshr(z, 8), 1024)
    return (((e + 15) << 10) | m).to(torch.int16)


def packed_dot_inputs(seed=PACKED.seed, records=128, outputs=2048, streams=64, device="cpu"):
    """fields int32 [records][outputs], scales binary16 bits [records][outputs],
    rhs f32 [records][streams][4] N(0,1), initial f32 [outputs] N(0,1)."""
    fields = _lshr(draws(seed, S_W, 0, records * outputs, device), 32).to(torch.int32).view(records, outputs)
    scales = f16_scales(seed, S_WSCALE, 0, records * outputs, device).view(records, outputs)
    rhs = normal(seed, S_X, 0, records * streams * 4, device).view(records, streams, 4)
    initial = normal(seed, S_INITIAL, 0, outputs, device)
    return fields, scales, rhs, initial


def routed_inputs(seed=ROUTED.seed, tokens=256, routes=8, hidden=1024, missing_percent=5, device="cpu"):
    """ids int32 [tokens][routes] uniform over num_rows = tokens * routes expert-output rows,
    missing_percent of them replaced by an out-of-range id (alternately -1 and num_rows + k);
    weights f32 [tokens][routes] uniform [1e-3, 1e-2); payload f32 [num_rows][hidden] N(0,1)."""
    num_rows = tokens * routes
    n = tokens * routes
    ids = randint(seed, S_LENGTHS, 0, n, 0, num_rows - 1, device)
    miss = randint(seed, S_COUNT, 0, n, 0, 99, device) < missing_percent
    odd = randint(seed, S_INITIAL, 0, n, 0, 1, device) == 1
    bad = torch.where(odd, torch.full_like(ids, -1), num_rows + randint(seed, S_XSCALE, 0, n, 0, 1000, device))
    ids = torch.where(miss, bad, ids).to(torch.int32).view(tokens, routes)
    weights = scales(seed, S_WSCALE, 0, n, device).view(tokens, routes)
    payload = torch.empty(num_rows, hidden, dtype=torch.float32, device=device)
    fill_chunked(payload, normal, seed, S_VALUES)
    return ids, weights, payload
