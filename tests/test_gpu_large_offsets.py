"""Inputs larger than 4 GiB: every kernel that walks a big operand is checked
on outputs whose data lies past the first 2^32 bytes, where a 32-bit byte
offset or element index would have wrapped.  The inputs are generated on the
device by the seeded generators; the sampled outputs are recomputed by the
CPU oracle from the same generators (or from host copies of the sampled
rows), to the same bar as the small parity tests: bit for bit for the integer
and in-order paths, within 1e-5 * sum|x| for the tree-reduced row sums.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32
REL_SUM = 1e-5


@pytest.fixture(scope="module")
def loom():
    import int8_dequant_dot_amd as m
    return m


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _np(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _late_rows(rows, row_bytes, extra, seed):
    """Row indices whose data starts past 4 GiB, plus the first and last rows."""
    first_late = -(-FOUR_GIB // row_bytes)
    assert first_late < rows
    rng = np.random.default_rng(seed)
    late = rng.integers(first_late, rows, extra)
    return np.unique(np.concatenate([[0, first_late - 1, first_late, rows - 1], late]))


# rows of 1024+ floats (a workgroup per row), 129-1023 (row tiles), 1-128 (rows packed per record)
@pytest.mark.parametrize("rows,cols", [(300_000, 4096), (2_200_000, 600), (12_000_000, 100)])
def test_row_sums_past_4gib(loom, device, rows, cols):
    x = synth.dense_matrix(synth.DENSE.seed, rows, cols, device=device)
    g = _np(loom.row_sums(x))
    sample = _late_rows(rows, 4 * cols, 40, seed=rows)
    xs = torch.cat([synth.dense_rows(synth.DENSE.seed, int(r), 1, cols) for r in sample])
    assert torch.equal(xs[-1].to(device), x[int(sample[-1])])
    del x
    ref, d, a = oracle.row_sums(xs.numpy())
    bound = REL_SUM * a + 1e-30
    assert np.all(np.abs(g[sample].astype(np.float64) - ref) <= bound), (rows, cols)
    assert np.all(np.abs(g[sample].astype(np.float64) - d) <= bound), (rows, cols)


def test_row_sums_one_row_past_4gib(loom, device):
    # one row of more than 2^30 floats: offsets inside the row pass 2^32 bytes
    cols = (1 << 30) + 1037
    x = torch.empty(1, cols, device=device)
    synth.fill_chunked(x, synth.uniform_pm1, synth.DENSE.seed, synth.S_VALUES)
    g = _np(loom.row_sums(x))
    host = x.cpu().numpy()
    del x
    ref, d, a = oracle.row_sums(host)
    bound = REL_SUM * a + 1e-30
    assert abs(float(g[0]) - float(ref[0])) <= bound[0] and abs(float(g[0]) - float(d[0])) <= bound[0]


@pytest.mark.parametrize("batch", [1, 8])
def test_i8_dequant_dot_past_4gib(loom, device, batch):
    rows, k = 600_000, 8192
    seed = synth.GEMV.seed if batch == 1 else synth.BATCHED.seed
    w = synth.i8_matrix(seed, synth.S_W, rows, k, device=device)
    x = synth.i8_rows(seed, synth.S_X, 0, batch, k)
    ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
    xs = synth.scales(seed, synth.S_XSCALE, 0, batch) if batch > 1 else None
    y, acc = loom.i8_dequant_dot(loom.pack_int8(w), ws.to(device), loom.pack_int8(x.to(device)),
                                 None if xs is None else xs.to(device), want_acc=True)
    gy, gacc = _np(y), _np(acc)
    sample = _late_rows(rows, k, 40, seed=batch)
    wsamp = torch.cat([synth.i8_rows(seed, synth.S_W, int(r), 1, k) for r in sample])
    assert torch.equal(wsamp[-1].to(device), w[int(sample[-1])])
    del w
    ry, racc = oracle.i8_dequant_dot(wsamp.numpy(), ws.numpy()[sample], x.numpy(),
                                     None if xs is None else xs.numpy())
    assert np.array_equal(gacc[sample], racc)
    assert np.array_equal(_bits(gy[sample]), _bits(ry))


def test_routed_combine_payload_past_4gib(loom, device):
    num_rows, hidden, tokens, routes = 1_200_000, 1024, 48, 8
    payload = torch.empty(num_rows, hidden, device=device)
    synth.fill_chunked(payload, synth.normal, synth.ROUTED.seed, synth.S_VALUES)
    first_late = FOUR_GIB // (4 * hidden)
    rng = np.random.default_rng(5)
    ids = rng.integers(first_late, num_rows, (tokens, routes))
    ids[0, :3] = [0, num_rows - 1, first_late - 1]
    ids[1, 2] = -1                               # a missing route
    ids[2, 5] = num_rows                         # one past the end: missing
    ids = torch.from_numpy(ids.astype(np.int32))
    weights = synth.scales(synth.ROUTED.seed, synth.S_WSCALE, 0, tokens * routes).view(tokens, routes)
    g = _np(loom.routed_combine(ids.to(device), weights.to(device), payload))
    # the oracle sees only the rows the routes name, renumbered in increasing order
    flat = ids.numpy().ravel()
    used = np.unique(flat[(flat >= 0) & (flat < num_rows)])
    rows = payload[torch.from_numpy(used).to(device)].cpu().numpy()
    del payload
    remap = np.full(flat.shape, -1, np.int32)
    ok = (flat >= 0) & (flat < num_rows)
    remap[ok] = np.searchsorted(used, flat[ok])
    ref = oracle.routed_combine(remap.reshape(tokens, routes), weights.numpy(), rows)[0]
    assert np.array_equal(_bits(g), _bits(ref))


def test_packed_dot_fields_past_4gib(loom, device):
    records, outputs, streams = 20, 1 << 26, 64   # fields 5 GiB, scales 2.5 GiB
    fields, scales, rhs, initial = synth.packed_dot_inputs(records=records, outputs=outputs, streams=streams,
                                                           device=device)
    g = _np(loom.packed_dot(fields, scales, rhs, records, initial))
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, outputs - 1], rng.integers(0, outputs, 60)]))
    idx = torch.from_numpy(sample).to(device)
    fs, ss = fields[:, idx].cpu().numpy(), scales[:, idx].cpu().numpy()
    # output i of the sampled problem reads stream i: give it the stream its original output read
    rs = rhs[:, torch.from_numpy(sample % streams).to(device)].cpu().numpy()
    init = initial[idx].cpu().numpy()
    del fields, scales
    ref = oracle.packed_dot(fs, ss, np.ascontiguousarray(rs), records, init)[0]
    assert np.array_equal(_bits(g[sample]), _bits(ref))


@pytest.mark.parametrize("cols", [2**31 - 4, 2**31 - 1])
def test_row_sums_one_row_of_nearly_2_31_floats(loom, device, cols):
    # the longest row the header admits, on the 128-bit path (cols % 4 == 0)
    # and on the 32-bit path: the record count of such a row must not
    # overflow 32-bit arithmetic
    x = torch.empty(1, cols, device=device)
    synth.fill_chunked(x, synth.uniform_pm1, synth.DENSE.seed, synth.S_VALUES)
    g = _np(loom.row_sums(x))
    host = x.cpu().numpy()
    del x
    ref, d, a = oracle.row_sums(host)
    bound = REL_SUM * a + 1e-30
    assert abs(float(g[0]) - float(ref[0])) <= bound[0] and abs(float(g[0]) - float(d[0])) <= bound[0], cols


def test_segment_sums_past_grid_limit(loom, device):
    # 2^26 + 5 segments of 4 columns: more one-wave segments than a grid of
    # fewer than 2^32 work-items holds, so some waves take two segments
    S, cols = 2**26 + 5, 4
    L = synth.randint(91, synth.S_LENGTHS, 0, S, 0, 2)
    off = synth.segment_offsets(L)
    total = int(off[-1])
    x = synth.segment_matrix(synth.SEGMENTS.seed, total, cols, device=device)
    cfg = loom.launch_config_invoke(loom.launch_config_lookup("segment_sums"), [S, cols, total])
    assert cfg["workgroups"][0] < S
    out, tails = loom.segment_sums(x, off.to(device))
    g, t = _np(out), _np(tails)
    ref, rtails, _, _ = oracle.segment_sums(x.cpu().numpy(), off.numpy(), shadows=False)
    assert np.array_equal(_bits(g), _bits(ref))
    assert np.array_equal(t, rtails)


def test_routed_combine_past_grid_limit(loom, device):
    # 2^26 + 3 tokens: some waves take two tokens
    tokens, routes, hidden, num_rows = 2**26 + 3, 1, 4, 1000
    ids = synth.randint(92, 1, 0, tokens * routes, -1, num_rows).view(tokens, routes).to(torch.int32)
    wts = synth.uniform_pm1(92, 2, 0, tokens * routes).view(tokens, routes)
    pay = synth.normal(92, 3, 0, num_rows * hidden).view(num_rows, hidden)
    cfg = loom.launch_config_invoke(loom.launch_config_lookup("routed_combine"), [tokens, routes, hidden])
    assert cfg["workgroups"][0] < tokens
    out = _np(loom.routed_combine(ids.to(device), wts.to(device), pay.to(device)))
    ref, _, _ = oracle.routed_combine(ids.numpy(), wts.numpy(), pay.numpy(), shadows=False)
    assert np.array_equal(_bits(out), _bits(ref))


@pytest.mark.parametrize("rows,k", [(20_000_000, 256), (3_000_000, 1536), (1_100_000, 4096), (400_000, 11008),
                                    (2**24 + 100, 8192)])
def test_i8_gemv_forms_past_4gib(loom, device, rows, k):
    # one vector in each GEMV form over more than 4 GiB of weights: rows packed
    # several to a record, groups of rows per record, a wave per block of rows,
    # a workgroup per row whose last record is partly empty, and a workgroup
    # per row of whole records (128 GiB) -- the last with more rows than a grid
    # of fewer than 2^32 work-items holds, so some workgroups take two rows
    if k == 8192:
        cfg = loom.launch_config_invoke(loom.launch_config_lookup("i8_dequant_dot"), [rows, k, 1])
        assert cfg["workgroup_size"][0] == 256 and cfg["workgroups"][0] < rows
    seed = synth.GEMV.seed
    w = synth.i8_matrix(seed, synth.S_W, rows, k, device=device)
    x = synth.i8_rows(seed, synth.S_X, 0, 1, k)
    ws = synth.scales(seed, synth.S_WSCALE, 0, rows)
    y, acc = loom.i8_dequant_dot(loom.pack_int8(w), ws.to(device), loom.pack_int8(x.to(device)), None,
                                 want_acc=True)
    gy, gacc = _np(y), _np(acc)
    sample = _late_rows(rows, k, 40, seed=k)
    sample = np.unique(np.concatenate([sample, np.arange(rows - 70, rows)]))
    wsamp = torch.cat([synth.i8_rows(seed, synth.S_W, int(r), 1, k) for r in sample])
    assert torch.equal(wsamp[-1].to(device), w[int(sample[-1])])
    del w
    ry, racc = oracle.i8_dequant_dot(wsamp.numpy(), ws.numpy()[sample], x.numpy(), None)
    assert np.array_equal(gacc[sample], racc)
    assert np.array_equal(_bits(gy[sample]), _bits(ry))
