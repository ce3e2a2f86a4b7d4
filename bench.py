"""Benchmark: achieved HBM GB/s of the streaming row sum and the int8 dequant dot on one MI355X.

One step is one pass of the whole hot path over resident synthetic inputs:
  1. row_sums        65536 x 4096 f32                        (1,074,003,968 B)
  2. i8_dequant_dot  16384 x 8192 int8 weights, 1 vector      (134,356,992 B, v_dot4)
  3. i8_dequant_dot  28672 x 8192 int8 weights, 8 vectors     (235,978,784 B, MFMA)
Bytes are algorithmic (each input read once, each output written once).  Every
input is a ring of copies rotated per step, so no launch finds its operands in
the 256 MB last-level cache: every launch reads HBM.

Prints one JSON line.  `value` is total algorithmic bytes per step / time per
step, timed over K back-to-back steps (phase A).  `roofline` is for the
dominant kernel (row_sums): its algorithmic bytes / its mean duration over five
repetitions of K back-to-back launches between two HIP events on the launch
stream (phase B; each start event queued behind one untimed launch, so the
timed ones never wait for the host).  `cpu_baseline` is
the CPU oracle on the same workload on one core (also used to check the outputs);
`cpu_baseline_all_cores` runs the same oracle calls over row blocks on every
usable host core.  `parts` gives each kernel's mean time and the median and
minimum of its five per-repetition means, and the same weights with 64
vectors (`i8_dequant_dot_batched_64`, outside the step); the
pages' own launch-bound shapes (the 63x32 tile, the 1009-element copy, the
guarded 63x32x4 rows, the 2048x128 packed dot, the 256-token routed combines)
add `us_graph`, the device time per call inside a HIP graph of back-to-back calls.

  python bench.py [--steps K] [--warmup W] [--no-segments] [--no-cpu] [--calibrate-copy MiB]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_OPS = 5.0e15  # dense int8 MFMA, MI355X
METRIC = "achieved HBM GB/s (and % of peak) for row-sum and int8 dequant-dot"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_row_sums_65536x4096.json")
KERNEL_SOURCES = ("device_common.hpp", "pipeline.hpp", "internal.hpp", "row_sums.hip")


def kernel_source_hash() -> str:
    """Hash of the row-sum kernel's sources with comments and blank space removed,
    so the recorded traffic stays valid across comment edits and lapses on any
    change to the code."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "int8_dequant_dot_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _bits(t):
    import torch
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _waves(cfg) -> int:
    """Waves along a launch's first grid axis (a split segment-sum launch runs one per part)."""
    return cfg["workgroups"][0] * cfg["workgroup_size"][0] // 64


def graph_us(fn, reps: int):
    """Device time of one call of `fn` (a launch-bound entry point), as
    (microseconds per call in a HIP graph of `reps` back-to-back calls,
    microseconds per eagerly issued call).  Between replays the outputs are
    poisoned by eager fills, and after each replay they must equal those of an
    eager call bit for bit."""
    import torch
    ref = [_bits(t).clone() for t in fn()]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) * 1e3 / reps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            res = fn()
    times = []
    for _ in range(5):
        for t in res:
            t.fill_(-7)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
        for t, r in zip(res, ref):
            if not torch.equal(_bits(t), r):
                raise RuntimeError("a graph replay gave a result that differs from the eager call")
    del g
    return sorted(times)[len(times) // 2], eager


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-segments", action="store_true",
                   help="skip the segment sums (16384 ragged segments, 34.5 GB)")
    p.add_argument("--segments", action="store_true", help=argparse.SUPPRESS)  # the default; kept for old commands
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run loom_copy_f32 over MIB MiB (counter calibration) and exit")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(every workload shards by independent rows; see the design notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import int8_dequant_dot_amd as loom
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        a = torch.ones(n, device=dev)
        b = torch.empty(n, device=dev)
        for _ in range(5):
            loom.copy_f32(a, b)
        torch.cuda.synchronize()
        log(f"copy_f32 calibration: {n} floats ({4 * n} B read, {4 * n} B written) x 5")
        return

    # ---------------------------------------------------------------- inputs (resident in HBM)
    # Each input is a ring of identical copies at different addresses, rotated
    # every step, so no launch finds its operands in the 256 MB last-level
    # cache whatever the loads' cache policy: row sums 2 x 1 GiB, GEMV
    # weights 4 x 128 MiB, batched weights 3 x 224 MiB.
    t0 = time.time()
    R2, C2 = 65536, 4096
    x2 = [synth.dense_matrix(synth.DENSE.seed, R2, C2, device=dev) for _ in range(2)]
    out2 = torch.empty(R2, device=dev)

    R4, K4 = 16384, 8192
    w4 = [synth.i8_matrix(synth.GEMV.seed, synth.S_W, R4, K4, device=dev) for _ in range(4)]
    x4 = synth.i8_matrix(synth.GEMV.seed, synth.S_X, 1, K4, device=dev)
    s4 = synth.scales(synth.GEMV.seed, synth.S_WSCALE, 0, R4, device=dev)
    out4 = torch.empty(R4, 1, device=dev)

    R5, K5, B5 = 28672, 8192, 8
    w5 = [synth.i8_matrix(synth.BATCHED.seed, synth.S_W, R5, K5, device=dev) for _ in range(3)]
    x5 = synth.i8_matrix(synth.BATCHED.seed, synth.S_X, B5, K5, device=dev)
    s5 = synth.scales(synth.BATCHED.seed, synth.S_WSCALE, 0, R5, device=dev)
    sx5 = synth.scales(synth.BATCHED.seed, synth.S_XSCALE, 0, B5, device=dev)
    out5 = torch.empty(R5, B5, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated in {time.time() - t0:.1f}s")

    w4p, x4p = [loom.pack_int8(w) for w in w4], loom.pack_int8(x4)
    w5p, x5p = [loom.pack_int8(w) for w in w5], loom.pack_int8(x5)
    bytes2 = R2 * C2 * 4 + R2 * 4
    bytes4 = R4 * K4 + K4 + R4 * 4 + R4 * 4
    bytes5 = R5 * K5 + B5 * K5 + R5 * 4 + B5 * 4 + R5 * B5 * 4
    step_bytes = bytes2 + bytes4 + bytes5

    kernels = [
        ("row_sums", bytes2, lambda i: loom.row_sums(x2[i % 2], out2)),
        ("i8_dequant_dot_gemv", bytes4, lambda i: loom.i8_dequant_dot(w4p[i % 4], s4, x4p, None, out=out4)),
        ("i8_dequant_dot_batched", bytes5, lambda i: loom.i8_dequant_dot(w5p[i % 3], s5, x5p, sx5, out=out5)),
    ]

    def step(i):
        for _, _, fn in kernels:
            fn(i)

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # Phase A: whole steps back to back, bracketed by two events.
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K
    log(f"timed {K} steps: {ms_per_step * 1e3:.1f} us/step")

    # Phase B: each kernel alone, K launches back to back (its input ring
    # still rotating) between two events on the launch stream: its mean
    # duration, with the event overhead amortised over K launches.  The start
    # event is queued behind one untimed launch of the same kernel (on the last
    # buffer of its ring), so the device is still busy when the host queues the
    # first timed launch: the timed launches run back to back, without the idle
    # gap of an empty queue waiting for the host's first call.
    # Five repetitions of the K launches give the median and minimum of the
    # per-launch mean; `us` is the mean over all five repetitions.
    REPS = 5
    per_kernel_ms, per_rep_ms = [], []
    for _, _, fn in kernels:
        reps = []
        for _ in range(REPS):
            torch.cuda.synchronize()
            fn(-1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(K):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / K)
        per_kernel_ms.append(sum(reps) / REPS)
        per_rep_ms.append(sorted(reps))

    parts = {}
    for (name, nbytes, _), ms, reps in zip(kernels, per_kernel_ms, per_rep_ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        parts[name] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "GB/s": round(gbs, 1),
                       "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                       "us_median": round(reps[REPS // 2] * 1e3, 2), "us_min": round(reps[0] * 1e3, 2)}
    # useful int8 operations of the batched product (2 per multiply-add) against
    # the dense int8 MFMA peak: the product is HBM-bound by a wide margin
    ops5 = 2 * R5 * K5 * B5
    parts["i8_dequant_dot_batched"]["TOP/s"] = round(ops5 / (per_kernel_ms[2] * 1e-3) / 1e12, 1)
    parts["i8_dequant_dot_batched"]["mfma_util"] = round(ops5 / (per_kernel_ms[2] * 1e-3) / INT8_PEAK_OPS, 4)

    # The same weights with 64 vectors (the column-tile kernel), outside the
    # step: five repetitions of K back-to-back launches, as above.
    B6 = 64
    x6p = loom.pack_int8(synth.i8_matrix(synth.BATCHED.seed, synth.S_X, B6, K5, device=dev))
    sx6 = synth.scales(synth.BATCHED.seed, synth.S_XSCALE, 0, B6, device=dev)
    out6 = torch.empty(R5, B6, device=dev)
    bytes6 = R5 * K5 + B6 * K5 + R5 * 4 + B6 * 4 + R5 * B6 * 4
    reps6 = []
    for _ in range(REPS):
        torch.cuda.synchronize()
        loom.i8_dequant_dot(w5p[2], s5, x6p, sx6, out=out6)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            loom.i8_dequant_dot(w5p[i % 3], s5, x6p, sx6, out=out6)
        e1.record(stream)
        torch.cuda.synchronize()
        reps6.append(e0.elapsed_time(e1) / K)
    ms6 = sum(reps6) / REPS
    reps6.sort()
    parts["i8_dequant_dot_batched_64"] = {
        "bytes": bytes6, "us": round(ms6 * 1e3, 2), "GB/s": round(bytes6 / (ms6 * 1e-3) / 1e9, 1),
        "frac_of_peak": round(bytes6 / (ms6 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "us_median": round(reps6[REPS // 2] * 1e3, 2), "us_min": round(reps6[0] * 1e3, 2),
        "TOP/s": round(2 * R5 * K5 * B6 / (ms6 * 1e-3) / 1e12, 1)}
    del x6p, out6

    if not args.no_segments:
        # The ragged segment sums: 16384 segments of U{0..4096} rows x 256
        # f32 columns (34.5 GB, far beyond the last-level cache), five
        # repetitions of back-to-back launches as above, then every output of
        # sampled segments checked bit for bit against the oracle on rows
        # regenerated on the host (each column is the in-order recurrence).
        S, CS = 16384, 256
        L = synth.segment_lengths(synth.SEGMENTS.seed, S, 4096, device=dev)
        off = synth.segment_offsets(L)
        total = int(off[-1].item())
        x3 = synth.segment_matrix(synth.SEGMENTS.seed, total, CS, device=dev)
        out3 = torch.empty(S, CS, device=dev)
        t3 = torch.empty(S, dtype=torch.int32, device=dev)
        bytes3 = total * CS * 4 + (S + 1) * 8 + S * CS * 4 + S * 4
        n3 = max(4, K // 5)
        reps3 = []
        for _ in range(REPS):
            torch.cuda.synchronize()
            loom.segment_sums(x3, off, out3, t3)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n3):
                loom.segment_sums(x3, off, out3, t3)
            e1.record(stream)
            torch.cuda.synchronize()
            reps3.append(e0.elapsed_time(e1) / n3)
        ms3 = sum(reps3) / REPS
        reps3.sort()
        gbs3 = bytes3 / (ms3 * 1e-3) / 1e9
        del x3
        torch.cuda.empty_cache()
        seg3 = (out3.cpu().numpy(), t3.cpu().numpy(), L.cpu().numpy(), off.cpu().numpy())

        # Few long segments (4 x 1,048,576 rows x 256 columns, 4 GiB): every
        # segment is split into parts summed in row order whose sums are added
        # in a fixed order (outside the step; parity in the tests).
        S4 = 4
        off4 = torch.arange(S4 + 1, dtype=torch.int64, device=dev) * (1 << 20)
        x34 = synth.segment_matrix(synth.SEGMENTS.seed, S4 << 20, CS, device=dev)
        out34 = torch.empty(S4, CS, device=dev)
        bytes34 = (S4 << 20) * CS * 4 + (S4 + 1) * 8 + S4 * CS * 4
        n34 = max(4, K // 5)
        reps34 = []
        for _ in range(REPS):
            torch.cuda.synchronize()
            loom.segment_sums(x34, off4, out34)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n34):
                loom.segment_sums(x34, off4, out34)
            e1.record(stream)
            torch.cuda.synchronize()
            reps34.append(e0.elapsed_time(e1) / n34)
        ms34 = sum(reps34) / REPS
        reps34.sort()
        parts["segment_sums_4x1M"] = {
            "bytes": bytes34, "us": round(ms34 * 1e3, 1), "GB/s": round(bytes34 / (ms34 * 1e-3) / 1e9, 1),
            "frac_of_peak": round(bytes34 / (ms34 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "us_median": round(reps34[REPS // 2] * 1e3, 1), "us_min": round(reps34[0] * 1e3, 1),
            "parts_per_segment": _waves(loom.launch_config_invoke(loom.launch_config_lookup("segment_sums"),
                                                                  [S4, CS, S4 << 20])) // S4}
        log(f"few long segments: {parts['segment_sums_4x1M']}")
        del x34, out34
        torch.cuda.empty_cache()
        parts["segment_sums"] = {"bytes": bytes3, "us": round(ms3 * 1e3, 1), "GB/s": round(gbs3, 1),
                                 "frac_of_peak": round(gbs3 / HBM_PEAK_GBS, 4),
                                 "us_median": round(reps3[REPS // 2] * 1e3, 1), "us_min": round(reps3[0] * 1e3, 1),
                                 "rows": total, "launches": REPS * n3}
        log(f"segment sums: {parts['segment_sums']}")
        del out3, t3

    # The pages' literal packed-dot recurrence: at the pages' own shape (2048
    # outputs x 128 records, latency-bound: microseconds per call) and at a
    # large shape (262144 outputs x 128 records) for bandwidth.
    # The large shape reads 192 MiB per call: two copies at different addresses,
    # alternated, keep it out of the last-level cache as the rings above do.
    for label, outputs in (("packed_dot_2048x128", 2048), ("packed_dot_262144x128", 262144)):
        ring = [synth.packed_dot_inputs(records=128, outputs=outputs, device=dev)
                for _ in range(2 if outputs > 2048 else 1)]
        pout = torch.empty(outputs, device=dev)
        nbytes = 128 * outputs * 6 + ring[0][2].numel() * 4 + 2 * outputs * 4

        def call(i, ring=ring, pout=pout):
            pf, ps, pr, pi = ring[i % len(ring)]
            loom.packed_dot(pf, ps, pr, 128, pi, out=pout)

        torch.cuda.synchronize()
        call(-1)  # untimed: the start event is queued behind it
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        del ring
        ms = e0.elapsed_time(e1) / K
        parts[label] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    # Routed row combine: the pages' n8/n32 shapes (1024-wide rows, latency-
    # bound) and a large one (16384 tokens x 8 routes) for bandwidth.
    for label, tokens, routes in (("routed_combine_n8_t256", 256, 8), ("routed_combine_n32_t256", 256, 32),
                                  ("routed_combine_n8_t16384", 16384, 8)):
        rid, rw, rp = synth.routed_inputs(tokens=tokens, routes=routes, hidden=1024, device=dev)
        rout = torch.empty(tokens, 1024, device=dev)
        valid = int(((rid >= 0) & (rid < rp.shape[0])).sum().item())
        nbytes = valid * (1024 * 4 + 4) + rid.numel() * 4 + tokens * 1024 * 4
        torch.cuda.synchronize()
        loom.routed_combine(rid, rw, rp, out=rout)  # untimed: the start event is queued behind it
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            loom.routed_combine(rid, rw, rp, out=rout)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / K
        parts[label] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del rid, rw, rp, rout

    # The pages' own shapes are launch-bound: a host call costs more than the
    # kernel.  Their device time per call comes from a HIP graph of back-to-back
    # calls; each replay is checked bit for bit against an eager call.
    tv, tc = synth.tile_inputs(device=dev)
    cin = synth.copy_inputs(device=dev)
    cout = torch.empty_like(cin)
    gv = synth.normal(1, synth.S_VALUES, 0, 63 * 32 * 4, dev).view(63, 32, 4)
    gout = torch.empty(32, device=dev)
    pf, ps, pr, pi = synth.packed_dot_inputs(records=128, outputs=2048, device=dev)
    pout = torch.empty(2048, device=dev)
    small = {
        "row_sum_tiles_63x32": (lambda: loom.row_sum_tiles(tv, tc), 63 * 32 * 4 + 32 * 4 + 8),
        "copy_f32_1009": (lambda: (loom.copy_f32(cin, out=cout),), 1009 * 8),
        "sum_guarded_rows_63x32x4": (lambda: (loom.sum_guarded_rows(gv, 63, 4, 32, out=gout),), 63 * 32 * 16 + 32 * 4),
        "packed_dot_2048x128": (lambda: (loom.packed_dot(pf, ps, pr, 128, pi, out=pout),), None),
    }
    for tokens, routes in ((256, 8), (256, 32)):
        rid, rw, rp = synth.routed_inputs(tokens=tokens, routes=routes, hidden=1024, device=dev)
        rout = torch.empty(tokens, 1024, device=dev)
        small[f"routed_combine_n{routes}_t{tokens}"] = (
            (lambda rid=rid, rw=rw, rp=rp, rout=rout: (loom.routed_combine(rid, rw, rp, out=rout),)), None)
    for label, (fn, nbytes) in small.items():
        us_graph, us_eager = graph_us(fn, max(K, 64))
        part = parts.setdefault(label, {"bytes": nbytes, "us": round(us_eager, 2)})
        part["us_graph"] = round(us_graph, 2)
        part["GB/s_graph"] = round(part["bytes"] / (us_graph * 1e-6) / 1e9, 1)
    del pf, ps, pr, pi

    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---------------------------------------------------------------- roofline of the dominant kernel
    achieved = parts["row_sums"]["GB/s"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("hbm_bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "row_sums 65536x4096 f32", "algorithmic_bytes": bytes2}

    # ---------------------------------------------------------------- CPU oracle baseline (+ output check)
    cpu = None
    cpu_all = None
    check = None
    if not args.no_cpu:
        import oracle
        hx2, hw4, hx4, hs4 = x2[0].cpu().numpy(), w4[0].cpu().numpy(), x4.cpu().numpy(), s4.cpu().numpy()
        hw5, hx5, hs5, hsx5 = w5[0].cpu().numpy(), x5.cpu().numpy(), s5.cpu().numpy(), sx5.cpu().numpy()
        passes, t_cpu = 0, 0.0
        while passes == 0 or t_cpu < 10.0:
            t = time.perf_counter()
            r2, _, a2 = oracle.row_sums(hx2, shadows=(passes == 0))
            r4, acc4 = oracle.i8_dequant_dot(hw4, hs4, hx4)
            r5, acc5 = oracle.i8_dequant_dot(hw5, hs5, hx5, hsx5)
            t_cpu += time.perf_counter() - t
            passes += 1
            if passes == 1:
                g2, g4, g5 = out2.cpu().numpy(), out4.cpu().numpy(), out5.cpu().numpy()
                err2 = float(np.max(np.abs(g2.astype(np.float64) - r2) / a2))
                err4 = float(np.max(np.abs(g4.astype(np.float64) - r4) / np.abs(r4)))
                err5 = float(np.max(np.abs(g5.astype(np.float64) - r5) / np.abs(r5)))
                check = {"row_sums_max_err_over_sum_abs": err2, "gemv_max_rel_err": err4,
                         "batched_max_rel_err": err5,
                         "pass": bool(err2 <= 1e-5 and err4 <= 2e-5 and err5 <= 2e-5)}
                log(f"oracle check: {check}")
        if not args.no_segments:
            # segment sums: every output of sampled segments, bit for bit (each
            # column is the in-order recurrence), on rows regenerated on the host
            g3, gt3, hL, hoff = seg3
            rng3 = np.random.default_rng(3)
            sample3 = np.unique(np.concatenate([[0, hL.size - 1, int(hL.argmax())], rng3.integers(0, hL.size, 5)]))
            same3 = bool(np.array_equal(gt3, (hL % 8).astype(np.int32)))
            for sg in sample3:
                b, e = int(hoff[sg]), int(hoff[sg + 1])
                ref3, _, _, _ = oracle.segment_sums(synth.segment_rows(synth.SEGMENTS.seed, b, e - b, 256).numpy(),
                                                    np.array([0, e - b]), shadows=False)
                same3 = same3 and bool(np.array_equal(g3[sg].view(np.uint32), ref3[0].view(np.uint32)))
            parts["segment_sums"]["oracle_check"] = {"segments": int(sample3.size), "rows": int(hL[sample3].sum()),
                                                     "bitwise_equal": same3}
            check["segment_sums_sampled_bitwise"] = same3
            check["pass"] = check["pass"] and same3
            log(f"segment sums oracle check: {parts['segment_sums']['oracle_check']}")
        cpu_gbs = passes * step_bytes / t_cpu / 1e9
        cpu = {"value": round(cpu_gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the full step (all three kernels' inputs and outputs), {passes} pass(es), "
                         f"{t_cpu:.1f}s, single-threaded C oracle"}

        # The same oracle calls over disjoint row blocks on every host core
        # this process may use (at most 16); ctypes drops the GIL for each
        # call, and each output's arithmetic is unchanged, so the results
        # must equal the single-threaded ones bit for bit.
        from concurrent.futures import ThreadPoolExecutor
        ncores = min(len(os.sched_getaffinity(0)), 16)

        def blocks(n):
            b = -(-n // ncores)
            return [(i, min(n, i + b)) for i in range(0, n, b)]

        def threaded_pass(pool):
            f2 = [pool.submit(oracle.row_sums, hx2[a:b], False) for a, b in blocks(hx2.shape[0])]
            f4 = [pool.submit(oracle.i8_dequant_dot, hw4[a:b], hs4[a:b], hx4) for a, b in blocks(hw4.shape[0])]
            f5 = [pool.submit(oracle.i8_dequant_dot, hw5[a:b], hs5[a:b], hx5, hsx5) for a, b in blocks(hw5.shape[0])]
            return (np.concatenate([f.result()[0] for f in f2]), np.concatenate([f.result()[0] for f in f4]),
                    np.concatenate([f.result()[0] for f in f5]))

        with ThreadPoolExecutor(ncores) as pool:
            tpasses, t_all = 0, 0.0
            while tpasses == 0 or t_all < 5.0:
                t = time.perf_counter()
                m2, m4, m5 = threaded_pass(pool)
                t_all += time.perf_counter() - t
                if tpasses == 0:
                    same = all(np.array_equal(u.view(np.uint32), v.view(np.uint32))
                               for u, v in ((m2, r2), (m4, r4), (m5, r5)))
                    if not same:
                        raise RuntimeError("threaded oracle differs from the single-threaded oracle")
                tpasses += 1
        cpu_all = {"value": round(tpasses * step_bytes / t_all / 1e9, 3), "unit": "GB/s", "cores": ncores,
                   "kind": "oracle",
                   "sample": f"the full step split into {ncores} row blocks per kernel, {tpasses} pass(es), "
                             f"{t_all:.1f}s; bitwise equal to the single-threaded run"}
        log(f"oracle on {ncores} cores: {cpu_all}")

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+int8(int32 acc)",
        "data": "synthetic (seeded SplitMix64, generated on the GPU)",
        "config": {"workload": "row_sums 65536x4096 f32 + i8_dequant_dot 16384x8192x1 + 28672x8192x8",
                   "bytes_per_step": step_bytes, "frac_of_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_all_cores": cpu_all,
        "parts": parts,
        "oracle_check": check,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
