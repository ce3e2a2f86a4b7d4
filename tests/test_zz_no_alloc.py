"""loom_segment_sums_noalloc (the call for callers that cannot allocate),
through the C ABI, against loom_segment_sums on the same inputs: two calls in
a row, the second with a smaller input, in a split launch (partials in the
library's static array), in a longest-first launch (its order index there)
and in a plain single-pass launch; the results must be the same bits, and
within the f32 tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def loom(device):
    import int8_dequant_dot_amd as m
    return m


def _call(lib, fn, x, off, cols):
    S = off.numel() - 1
    out = torch.full((S, cols), float("nan"), device=x.device)
    tails = torch.full((S,), -7, dtype=torch.int32, device=x.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = getattr(lib, fn)(ctypes.c_void_p(x.data_ptr()), x.shape[0], ctypes.c_void_p(off.data_ptr()), S, cols,
                          ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(tails.data_ptr()), stream)
    assert st == 0, (fn, st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), tails.cpu().numpy()


# (lengths, cols) of the two calls; the second is smaller than the first
# (fewer rows, segments and columns)
CALLS = {
    # parts in runs of 8 (up to 512 columns), then a part per partial (wider
    # rows), then runs again on a smaller input
    "split": [([100000, 5, 60000], 256), ([40000, 7, 20000], 1000), ([30000, 20000], 100)],
    # 2 to 2^15 segments averaging >= 512 rows, >= 2^26 floats
    "longest_first": [([1300, 0, 37, 900] * 80, 512), ([9, 1500] * 95, 480)],
    "single": [([300, 0, 37, 900] * 100, 260), ([9, 400] * 150, 64)],
}


@pytest.mark.parametrize("mode", list(CALLS))
def test_noalloc_matches_segment_sums(loom, device, mode):
    lib = loom.library()
    seg = loom.launch_config_lookup("segment_sums")
    for lengths, cols in CALLS[mode]:
        L = torch.tensor(lengths, dtype=torch.int64)
        off = synth.segment_offsets(L)
        total = int(off[-1])
        cfg = loom.launch_config_invoke(seg, [len(lengths), cols, total])
        parts = cfg["workgroups"][0] * (cfg["workgroup_size"][0] // 64) // len(lengths)  # a wave per part
        assert (parts > 1) == (mode == "split"), parts
        if mode != "split":
            ordered = total // len(lengths) >= 512 and total * cols >= 2 ** 26
            assert ordered == (mode == "longest_first"), (total, cols)
        x = synth.segment_rows(synth.SEGMENTS.seed, 0, total, cols)
        dx, doff = x.to(device), off.to(device)
        g_na, t_na = _call(lib, "loom_segment_sums_noalloc", dx, doff, cols)
        g, t = _call(lib, "loom_segment_sums", dx, doff, cols)
        assert np.array_equal(g_na.view(np.uint32), g.view(np.uint32)), (lengths[:4], cols)
        assert np.array_equal(t_na, t)
        ref, rt, d, a = oracle.segment_sums(x.numpy(), off.numpy())
        bound = 1e-5 * a + 1e-30
        assert np.all(np.abs(g_na.astype(np.float64) - ref) <= bound)
        assert np.all(np.abs(g_na.astype(np.float64) - d) <= bound)
        assert np.array_equal(t_na, rt)
