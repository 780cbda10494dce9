"""GPU parity at the largest sizes: calls whose per-buffer extent passes the
2 GiB a single launch may address (so the host splits them into launches
over contiguous spans, row bands or pieces of one long row, and the ring
into windows), and the runtime rank-count kernel at N = 64 on 64 MiB
buffers.

Inputs are drawn on the device (seeded; ``workloads.draw_device``).  The
i32 sums wrap and do not depend on the fold order, so those results are
checked whole against the wrapped sum that torch computes on the device;
every case is also checked on sampled windows -- around every launch split,
at both ends and at random positions -- against the oracle, element by
element, from the inputs read back at the same positions.
"""

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W
from tests.gpu_helpers import compare, say

pytestmark = pytest.mark.gpu

GIB2 = 1 << 31
RECIPE = {"f32": "uniform_pm1", "bf16": "normal_1e-2", "f16": "normal_sat", "i32": "int_pm2^20"}
NP_BITS = {"f32": np.float32, "i32": np.int32, "bf16": np.uint16, "f16": np.uint16}
ES = {"f32": 4, "i32": 4, "bf16": 2, "f16": 2}
PAD = 64  # sentinel elements after every dst


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _sources(dtype, n, nranks, seed):
    return [W.draw_device(RECIPE[dtype], n, seed + r) for r in range(nranks)]


def _sentinel_dev(dtype, n):
    t = torch.empty(n, dtype=torch.int32 if ES[dtype] == 4 else torch.int16, device="cuda")
    t.fill_(-1)  # all-ones bits
    return t


def _gather(t, idx, dtype):
    """Elements of a raw-bits device tensor at host indices, in the oracle's
    storage type."""
    return t[torch.from_numpy(idx).to("cuda")].cpu().numpy().view(NP_BITS[dtype])


def _samples(n, splits, rng, k=2048, w=64):
    """Indices: windows of +-w around each split, both ends, k random."""
    parts = [np.arange(0, min(w, n)), np.arange(max(0, n - w), n),
             rng.integers(0, n, k)]
    for b in splits:
        parts.append(np.arange(max(0, b - w), min(n, b + w)))
    return np.unique(np.concatenate(parts)).astype(np.int64)


def _check_samples(srcs, dst, idx, dtype, op, root):
    got = _gather(dst, idx, dtype)
    ins = [np.ascontiguousarray(_gather(s, idx, dtype)) for s in srcs]
    want = W.sentinel_buffer(dtype, idx.size)
    oracle.treduce(ins, want, root=root, dtype=dtype, op=op, rows=1, cols=idx.size,
                   ld=idx.size, valid_rows=1, valid_cols=idx.size)
    ok = compare(dtype, got, want)
    assert ok.all(), (int(idx[~ok][0]), int(np.count_nonzero(~ok)))


def _wrapped_sum(srcs):
    """Sum of i32 tensors modulo 2^32, in two's complement (order-free)."""
    acc = torch.zeros(srcs[0].numel(), dtype=torch.int64, device="cuda")
    for s in srcs:
        acc += s.to(torch.int64)
    return (torch.remainder(acc + (1 << 31), 1 << 32) - (1 << 31)).to(torch.int32)


def _plan(srcs, nranks, root, dst, rows, cols, ld, vr, vc, dtype, op):
    st, info = B.ptored_treduce_plan([s.data_ptr() for s in srcs], nranks, root, dst, rows, cols,
                                     ld, vr, vc, B.DTYPES[dtype], B.OPS[op])
    assert st == 0
    return info


@pytest.mark.parametrize("dtype,op", [("i32", "sum"), ("bf16", "sum")])
def test_contiguous_span_over_2gib(dtype, op):
    n = GIB2 // ES[dtype] + 4099  # 2 GiB + 4099 elements per buffer
    say(f"large span {dtype} {op} count={n}")
    srcs = _sources(dtype, n, 2, 7100)
    dst = _sentinel_dev(dtype, n + PAD)
    info = _plan(srcs, 2, 1, dst.data_ptr(), 1, n, n, 1, n, dtype, op)
    assert info.launches == 2
    st = B.ptored_treduce([s.data_ptr() for s in srcs], 2, 1, dst.data_ptr(), 1, n, n, 1, n,
                          B.DTYPES[dtype], B.OPS[op], _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    assert bool((dst[n:] == -1).all())
    if dtype == "i32":
        assert bool((dst[:n] == _wrapped_sum(srcs)).all())
    rng = np.random.default_rng(7101)
    _check_samples(srcs, dst, _samples(n, [GIB2 // ES[dtype]], rng), dtype, op, root=1)


def test_row_bands_over_2gib():
    """f32 max, N = 3, rows of 16400 with 16397 valid: 2.16 GB of extent,
    cut into two row bands."""
    dtype, op, nr = "f32", "max", 3
    rows, ld, vr, vc = 33000, 16400, 32999, 16397
    size = rows * ld
    say(f"large row bands {dtype} {op} {rows}x{ld} valid {vr}x{vc}")
    srcs = _sources(dtype, size, nr, 7200)
    dst = _sentinel_dev(dtype, size)
    info = _plan(srcs, nr, 2, dst.data_ptr(), rows, ld, ld, vr, vc, dtype, op)
    assert info.launches == 2
    st = B.ptored_treduce([s.data_ptr() for s in srcs], nr, 2, dst.data_ptr(), rows, ld, ld, vr,
                          vc, B.DTYPES[dtype], B.OPS[op], _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    d2 = dst.view(rows, ld)
    assert bool((d2[:, vc:] == -1).all()) and bool((d2[vr:, :] == -1).all())
    rpl = (GIB2 - vc * 4) // (ld * 4) + 1  # rows per band, as the host cuts them
    rng = np.random.default_rng(7201)
    band_rows = [rpl - 1, rpl, 0, vr - 1] + list(rng.integers(0, vr, 6))
    idx = np.concatenate([r * ld + np.arange(vc) for r in band_rows]).astype(np.int64)
    _check_samples(srcs, dst, np.unique(idx), dtype, op, root=2)


def test_rows_longer_than_one_launch():
    """f16 sum, two rows of 2 GiB + 80 bytes each (37 of the last 40
    elements valid): every row is cut into two spans."""
    dtype, op = "f16", "sum"
    cols = GIB2 // 2 + 40
    rows, ld, vr, vc = 2, cols, 2, cols - 3
    size = rows * ld
    say(f"large long rows {dtype} {op} {rows}x{ld} valid {vr}x{vc}")
    srcs = _sources(dtype, size, 2, 7300)
    dst = _sentinel_dev(dtype, size)
    info = _plan(srcs, 2, 0, dst.data_ptr(), rows, cols, ld, vr, vc, dtype, op)
    assert info.launches == 4
    st = B.ptored_treduce([s.data_ptr() for s in srcs], 2, 0, dst.data_ptr(), rows, cols, ld, vr,
                          vc, B.DTYPES[dtype], B.OPS[op], _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    d2 = dst.view(rows, ld)
    assert bool((d2[:, vc:] == -1).all())
    rng = np.random.default_rng(7301)
    per = GIB2 // 2
    idx = np.concatenate([r * ld + _samples(vc, [per], rng) for r in range(rows)])
    _check_samples(srcs, dst, idx, dtype, op, root=0)


def test_allreduce_over_2gib():
    dtype, op, nr = "i32", "sum", 2
    n = GIB2 // 4 + 4099
    say(f"large allreduce {dtype} {op} count={n}")
    bufs = _sources(dtype, n, nr, 7400)
    before = [b.clone() for b in bufs]
    want = _wrapped_sum(before)
    st = B.ptored_allreduce([b.data_ptr() for b in bufs], nr, 0, 1, n, n, 1, n,
                            B.DTYPES[dtype], B.OPS[op], None, _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    for b in bufs:
        assert bool((b == want).all())
    rng = np.random.default_rng(7401)
    _check_samples(before, bufs[1], _samples(n, [GIB2 // 4], rng), dtype, op, root=0)


def test_reduce_scatter_ring_over_2gib():
    """i32 sum, N = 3, 3.2 GB streams: two windows; every segment checked
    whole, and untouched outside its segment."""
    dtype, op, nr = "i32", "sum", 3
    count = 3 * (1 << 28) + 5
    say(f"large ring {dtype} {op} N={nr} count={count}")
    srcs = _sources(dtype, count, nr, 7500)
    dsts = [_sentinel_dev(dtype, count) for _ in range(nr)]
    st = B.ptored_reduce_scatter_ring([s.data_ptr() for s in srcs], nr,
                                      [d.data_ptr() for d in dsts], count, B.DTYPES[dtype],
                                      B.OPS[op], None, _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    bounds = oracle.ring_bounds(count, nr, dtype)
    want = _wrapped_sum(srcs)
    for s in range(nr):
        lo, hi = int(bounds[s]), int(bounds[s + 1])
        assert bool((dsts[s][lo:hi] == want[lo:hi]).all()), s
        assert bool((dsts[s][:lo] == -1).all()) and bool((dsts[s][hi:] == -1).all()), s
    # sampled windows against the oracle's ring-order fold, around the window split
    rng = np.random.default_rng(7501)
    for s in range(nr):
        lo, hi = int(bounds[s]), int(bounds[s + 1])
        idx = lo + _samples(hi - lo, [GIB2 // 4 - lo] if lo < GIB2 // 4 < hi else [], rng, k=512)
        ring = [srcs[(s + 1 + k) % nr] for k in range(nr)]
        _check_samples(ring, dsts[s], idx, dtype, op, root=0)


def test_accumulate_add_over_2gib():
    dtype, nr = "i32", 2
    n = GIB2 // 4 + 4099
    say(f"large accumulate {dtype} count={n}")
    srcs = _sources(dtype, n, nr, 7600)
    dst = W.draw_device(RECIPE[dtype], n, 7699)
    want = _wrapped_sum(srcs + [dst.clone()])
    st = B.ptored_accumulate_add([s.data_ptr() for s in srcs], nr, dst.data_ptr(), 1, n, n, 1,
                                 n, B.DTYPES[dtype], None, _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    assert bool((dst == want).all())


@pytest.mark.parametrize("skip", [1, 132])
def test_common_lead_full_size(skip):
    """n16_i32_4096x4096 with every buffer `skip` elements past its allocation's
    start (4 bytes: a head in the first 16-byte block; 528 bytes: 33 skipped
    slots before it, numbered from the 1 KiB boundary): whole result against
    the wrapped sum, sampled windows against the oracle."""
    w = W.WORKLOADS["n16_i32_4096x4096"]
    n = w.buffer_elems
    say(f"large common offset n16_i32_4096x4096 +{4 * skip} bytes")
    raw = _sources("i32", n + skip, w.nranks, 7800)  # spare elements in front of each
    srcs = [t[skip:] for t in raw]
    dbuf = _sentinel_dev("i32", n + skip + PAD)
    dst = dbuf[skip:]
    st, info = B.ptored_treduce_plan([t.data_ptr() for t in srcs], w.nranks, 0, dst.data_ptr(),
                                     w.rows, w.cols, w.ld, w.valid_rows, w.valid_cols,
                                     B.DTYPES["i32"], B.OPS["sum"])
    assert st == 0 and B.PATHS[info.path] == "vec_fixed"
    if all(t.data_ptr() % 1024 == 4 * skip % 1024 for t in srcs + [dst]):
        assert info.lead == 4 * skip
    st = B.ptored_treduce([t.data_ptr() for t in srcs], w.nranks, 0, dst.data_ptr(), w.rows,
                          w.cols, w.ld, w.valid_rows, w.valid_cols, B.DTYPES["i32"],
                          B.OPS["sum"], _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    assert bool((dst[:n] == _wrapped_sum([t[:n] for t in srcs])).all())
    assert bool((dbuf[:skip] == -1).all()) and bool((dst[n:] == -1).all())
    rng = np.random.default_rng(7801)
    _check_samples(srcs, dst, _samples(n, [], rng), "i32", "sum", root=0)


@pytest.mark.parametrize("dtype,op", [("f32", "sum"), ("bf16", "max")])
def test_n64_full_size(dtype, op):
    """N = 64 (the largest rank count) on 64 MiB buffers: the runtime rank
    loop at full size, root in the middle."""
    nr, rows = 64, 4096
    cols = (1 << 26) // ES[dtype] // rows
    n = rows * cols
    say(f"large N=64 {dtype} {op} {rows}x{cols}")
    srcs = _sources(dtype, n, nr, 7700)
    dst = _sentinel_dev(dtype, n + PAD)
    st = B.ptored_treduce([s.data_ptr() for s in srcs], nr, 37, dst.data_ptr(), rows, cols, cols,
                          rows, cols, B.DTYPES[dtype], B.OPS[op], _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    assert bool((dst[n:] == -1).all())
    rng = np.random.default_rng(7701)
    _check_samples(srcs, dst, _samples(n, [], rng, k=4096), dtype, op, root=37)
