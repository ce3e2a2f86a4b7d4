"""Every entry point inside a captured HIP graph.

A launch sequence that is captured once and replayed must give, on every
replay, the bits of the same call issued eagerly: the entry points enqueue
kernels only (no host synchronisation, allocation or memset on the stream),
and no kernel depends on state left by an earlier launch.  Between replays
the outputs are poisoned and unrelated eager work runs on the same stream.
One case per kernel variant (narrow, tiled and long-row row sums; GEMV and
all three MFMA kernels; one-output and four-output packed dot; ...).  The
segment sums' split and longest-first launches, whose workspace the
allocating call takes from the stream-ordered allocator, are captured
through the no-alloc entry point, the one meant for graphs.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def loom():
    import int8_dequant_dot_amd as m
    return m


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _cases(loom, dev):
    c = {}
    x = synth.copy_inputs(device=dev)
    cout = torch.full((1024,), -1.0, device=dev)
    c["copy_f32"] = lambda: (loom.copy_f32(x, cout[:1009]),)
    tv = synth.normal(1, synth.S_VALUES, 0, 63 * 32, dev).view(63, 32)
    ti = synth.normal(1, synth.S_INITIAL, 0, 32, dev)
    c["row_sum_tiles"] = lambda: loom.row_sum_tiles(tv, 45, ti)
    for name, (rows, cols) in {"row_sums_narrow": (5000, 37), "row_sums_tiled": (3000, 600),
                               "row_sums_long": (300, 4096)}.items():
        xr = synth.dense_rows(synth.DENSE.seed, 0, rows, cols, dev)
        o = torch.empty(rows, device=dev)
        c[name] = (lambda xr=xr, o=o: (loom.row_sums(xr, o),))
    for cols in (256, 300):
        off = synth.segment_offsets(torch.tensor([0, 5, 100, 17, 8, 0, 33], dtype=torch.int64)).to(dev)
        xs = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), cols, dev)
        so = torch.empty(7, cols, device=dev)
        st = torch.empty(7, dtype=torch.int32, device=dev)
        c[f"segment_sums_{cols}"] = (lambda xs=xs, off=off, so=so, st=st: loom.segment_sums(xs, off, so, st))
    # few long segments (split: partials in the static array) and many long
    # uneven ones over >= 2^26 floats (longest first: the order index there)
    for name, L, cols in (("split", torch.tensor([40000, 3, 30000], dtype=torch.int64), 256),
                          ("ordered", torch.cat([torch.tensor([40000, 0], dtype=torch.int64),
                                                 synth.segment_lengths(78, 298, 1600)]), 256)):
        off = synth.segment_offsets(L).to(dev)
        xs = synth.segment_rows(synth.SEGMENTS.seed, 0, int(off[-1]), cols, dev)
        so = torch.empty(L.numel(), cols, device=dev)
        st = torch.empty(L.numel(), dtype=torch.int32, device=dev)
        c[f"segment_sums_noalloc_{name}"] = (lambda xs=xs, off=off, so=so, st=st:
                                             loom.segment_sums(xs, off, so, st, noalloc=True))
    for batch in (1, 8, 16, 40):
        w = loom.pack_int8(synth.i8_rows(5, synth.S_W, 0, 300, 8192, dev))
        v = loom.pack_int8(synth.i8_rows(5, synth.S_X, 0, batch, 8192, dev))
        ws = synth.scales(5, synth.S_WSCALE, 0, 300, dev)
        vs = synth.scales(5, synth.S_XSCALE, 0, batch, dev)
        y = torch.empty(300, batch, device=dev)
        a = torch.empty(300, batch, dtype=torch.int32, device=dev)
        c[f"i8_dequant_dot_b{batch}"] = (lambda w=w, v=v, ws=ws, vs=vs, y=y, a=a:
                                         loom.i8_dequant_dot(w, ws, v, vs, y, a, want_acc=True))
    # 4 vectors at k = 1024: one wave per 16-row tile
    wk = loom.pack_int8(synth.i8_rows(7, synth.S_W, 0, 300, 1024, dev))
    vk = loom.pack_int8(synth.i8_rows(7, synth.S_X, 0, 4, 1024, dev))
    wsk = synth.scales(7, synth.S_WSCALE, 0, 300, dev)
    yk = torch.empty(300, 4, device=dev)
    ak = torch.empty(300, 4, dtype=torch.int32, device=dev)
    c["i8_dequant_dot_b4_k1024"] = lambda: loom.i8_dequant_dot(wk, wsk, vk, None, yk, ak, want_acc=True)
    # 64 vectors over 5000 rows: two row tiles per wave in the column-tile kernel
    wt = loom.pack_int8(synth.i8_rows(6, synth.S_W, 0, 5000, 1024, dev))
    vt = loom.pack_int8(synth.i8_rows(6, synth.S_X, 0, 64, 1024, dev))
    wst = synth.scales(6, synth.S_WSCALE, 0, 5000, dev)
    vst = synth.scales(6, synth.S_XSCALE, 0, 64, dev)
    yt = torch.empty(5000, 64, device=dev)
    at = torch.empty(5000, 64, dtype=torch.int32, device=dev)
    c["i8_dequant_dot_b64_5000"] = lambda: loom.i8_dequant_dot(wt, wst, vt, vst, yt, at, want_acc=True)
    for outputs, records in ((2048, 128), (65536 + 320, 12)):
        f, s, r, i = synth.packed_dot_inputs(records=records, outputs=outputs, device=dev)
        po = torch.empty(outputs, device=dev)
        c[f"packed_dot_{outputs}"] = (lambda f=f, s=s, r=r, i=i, po=po, n=records:
                                      (loom.packed_dot(f, s, r, n, i, po),))
    gv = synth.normal(1, synth.S_VALUES, 0, 63 * 32 * 4, dev).view(63, 32, 4)
    go = torch.empty(32, device=dev)
    c["sum_guarded_rows"] = lambda: (loom.sum_guarded_rows(gv, 61, 3, 29, go),)
    ids, wts, pay = synth.routed_inputs(tokens=64, routes=8, hidden=1024, device=dev)
    ro = torch.empty(64, 1024, device=dev)
    c["routed_combine"] = lambda: (loom.routed_combine(ids, wts, pay, ro),)
    return c


CASE_NAMES = ["copy_f32", "row_sum_tiles", "row_sums_narrow", "row_sums_tiled", "row_sums_long",
              "segment_sums_256", "segment_sums_300", "segment_sums_noalloc_split", "segment_sums_noalloc_ordered",
              "i8_dequant_dot_b1", "i8_dequant_dot_b8", "i8_dequant_dot_b16",
              "i8_dequant_dot_b40", "i8_dequant_dot_b64_5000", "i8_dequant_dot_b4_k1024",
              "packed_dot_2048", "packed_dot_65856", "sum_guarded_rows", "routed_combine"]


@pytest.fixture(scope="module")
def cases(loom, device):
    c = _cases(loom, device)
    assert sorted(c) == sorted(CASE_NAMES)
    return c


@pytest.mark.parametrize("name", CASE_NAMES)
def test_graph_replays_match_eager(loom, device, cases, name):
    fn = cases[name]
    ref = [_bits(t).clone() for t in fn()]
    torch.cuda.synchronize()
    # warm up on a side stream (default priority) before capturing, as torch recommends
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    scratch_in = torch.arange(4096, dtype=torch.float32, device=device)
    scratch_out = torch.empty_like(scratch_in)
    for replay in range(4):
        for t in res:
            t.fill_(-7)                                   # poison the graph's outputs eagerly
        loom.copy_f32(scratch_in, scratch_out)            # unrelated eager work on the same stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(res, ref):
            assert torch.equal(_bits(t), r), (name, replay)
        assert torch.equal(scratch_out, scratch_in)
    del g
