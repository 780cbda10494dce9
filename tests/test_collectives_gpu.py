"""GPU parity of the collective variants through the C ABI: in-place
allreduce, the ring reduce-scatter share, and push-with-add accumulation.

Bar: bit-exact for the allreduce and the reduce-scatter (same fold order and
arithmetic as the oracle); for push-with-add here, bit-exact for i32, and for
the float types within the rounding bound of N additions in any order,
N * u * sum|x| (u the unit roundoff; an addition whose result is subnormal is
exact, and the atomics keep subnormals, so no absolute slack is needed).  The
exact checks of push-with-add are in test_push_gpu.py.
"""

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W
from tests.gpu_helpers import DevBuf, ESIZE, compare, isnan_bits, bits, say, sentinel, valid_mask
from tests.test_parity_gpu import _rand_elems

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "max", "min", "prod"]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _upload(arrs, offs, fill=0xA5):
    out = []
    for a, o in zip(arrs, offs):
        b = DevBuf(a.size * a.itemsize, o, fill=fill)
        b.upload(a)
        out.append(b)
    return out


# ------------------------------------------------------------- allreduce ---

@pytest.mark.parametrize("dtype", DT)
def test_allreduce_in_place_random(dtype):
    rng = np.random.default_rng({"f32": 31, "bf16": 32, "f16": 33, "i32": 34}[dtype])
    es = ESIZE[dtype]
    for case in range(24):
        n = int(rng.choice([2, 3, 5, 8, 16, 17, 40]))
        rows = int(rng.integers(1, 40))
        cols = int(rng.integers(1, 600))
        ld = cols + int(rng.choice([0, 0, 3, 8]))
        vr, vc = int(rng.integers(1, rows + 1)), int(rng.integers(1, cols + 1))
        root = int(rng.integers(0, n))
        op = OPS[case % 4]
        flags = [0, B.PTORED_FORCE_ELEMENTWISE, B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES,
                 B.PTORED_FORCE_RUNTIME_N, B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK,
                 B.PTORED_FULL_OCCUPANCY][case % 6]
        offs = [0 if case % 3 else int(rng.integers(0, 8)) * es for _ in range(n)]
        size = (rows - 1) * ld + cols
        srcs = [_rand_elems(dtype, rng, size, wild=0.05) for _ in range(n)]
        bufs = _upload(srcs, offs)
        say(f"allreduce#{case} {dtype} {op} N={n} root={root} {rows}x{cols} ld={ld} "
            f"valid={vr}x{vc} flags={flags}")
        st = B.ptored_allreduce([b.ptr for b in bufs], n, root, rows, cols, ld, vr, vc,
                                B.DTYPES[dtype], B.OPS[op], B.tuning(flags=flags), _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = [s.copy() for s in srcs]
        oracle.allreduce_inplace(want, root=root, dtype=dtype, op=op, rows=rows, cols=cols,
                                 ld=ld, valid_rows=vr, valid_cols=vc)
        m = valid_mask(rows, ld, vr, vc, size)
        for r, b in enumerate(bufs):
            got = b.download(dtype)
            assert compare(dtype, got[m], want[r][m]).all(), (case, r)
            assert np.array_equal(got[~m].view(np.uint8), srcs[r][~m].view(np.uint8)), (case, r)
            assert b.guards_intact()


@pytest.mark.parametrize("dtype", DT)
def test_collectives_common_lead(dtype):
    """Allreduce, ring reduce-scatter and push-with-add over buffers that all
    start the same number of bytes past a 16-byte boundary, in every other
    case at one offset within a 128-byte line."""
    rng = np.random.default_rng({"f32": 61, "bf16": 62, "f16": 63, "i32": 64}[dtype])
    es = ESIZE[dtype]
    for case in range(12):
        lead = int(rng.choice(list(range(es, 16, es))))
        n = int(rng.choice([2, 5, 8, 16]))
        rows, cols = int(rng.integers(2, 30)), int(rng.integers(16, 900))
        ld = cols + (-cols) % 8 + 8 * int(rng.integers(0, 2))
        vr, vc = int(rng.integers(1, rows + 1)), int(rng.integers(8, cols + 1))
        size = (rows - 1) * ld + cols
        op = OPS[case % 4]
        if case % 2:  # one offset within a 128-byte line for every buffer
            common = lead + 16 * int(rng.integers(0, 8))
            offs = [common] * n
            doff = lambda: common  # noqa: E731
        else:  # one offset within a 16-byte block only
            offs = [lead + 16 * int(rng.integers(0, 3)) for _ in range(n)]
            doff = lambda: lead + 16 * int(rng.integers(0, 3))  # noqa: E731
        say(f"lead collectives#{case} {dtype} {op} lead={lead} N={n} {rows}x{cols} ld={ld} "
            f"valid={vr}x{vc}")
        # allreduce in place
        srcs = [_rand_elems(dtype, rng, size, wild=0.05) for _ in range(n)]
        bufs = _upload(srcs, offs)
        st = B.ptored_allreduce([b.ptr for b in bufs], n, case % n, rows, cols, ld, vr, vc,
                                B.DTYPES[dtype], B.OPS[op], None, _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = [x.copy() for x in srcs]
        oracle.allreduce_inplace(want, root=case % n, dtype=dtype, op=op, rows=rows, cols=cols,
                                 ld=ld, valid_rows=vr, valid_cols=vc)
        for b, w_ in zip(bufs, want):
            assert compare(dtype, b.download(dtype), w_).all(), case
            assert b.guards_intact()
        # ring reduce-scatter over the whole stream
        count = size
        sb = _upload(srcs, offs)
        db = [DevBuf(count * es, doff(), fill=0xFF) for _ in range(n)]
        st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], n, [b.ptr for b in db], count,
                                          B.DTYPES[dtype], B.OPS[op], None, _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = [sentinel(dtype, count) for _ in range(n)]
        oracle.reduce_scatter_ring([x.copy() for x in srcs], want, count=count, dtype=dtype,
                                   op=op)
        for b, w_ in zip(db, want):
            assert compare(dtype, b.download(dtype), w_).all(), case
            assert b.guards_intact()
        # push-with-add (i32 exact; floats within the bound of N additions)
        fsrcs = [_finite_values(dtype, rng, size) for _ in range(n)]
        d0 = _finite_values(dtype, rng, size)
        sb = _upload(fsrcs, offs)
        dd = _upload([d0], [doff()])[0]
        st = B.ptored_accumulate_add([b.ptr for b in sb], n, dd.ptr, rows, cols, ld, vr, vc,
                                     B.DTYPES[dtype], None, _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        got = dd.download(dtype)
        wacc = d0.copy()
        exact, absum = oracle.accumulate_add(fsrcs, wacc, dtype=dtype, rows=rows, cols=cols,
                                             ld=ld, valid_rows=vr, valid_cols=vc)
        m = valid_mask(rows, ld, vr, vc, size)
        assert np.array_equal(got[~m].view(np.uint8), d0[~m].view(np.uint8)), case
        if dtype == "i32":
            assert compare(dtype, got[m], wacc[m]).all(), case
        else:
            g = oracle.to_double(dtype, bits(dtype, got[m]).astype(np.uint32))
            bound = n * UNIT[dtype] * absum * 1.0001
            assert np.all(np.abs(g - exact) <= bound), case


def test_allreduce_two_entries_same_buffer():
    """The same buffer listed twice counts as two ranks and gets the result."""
    rng = np.random.default_rng(35)
    a = rng.standard_normal(4096).astype(np.float32)
    c = rng.standard_normal(4096).astype(np.float32)
    ba, bc = _upload([a, c], [0, 0])
    st = B.ptored_allreduce([ba.ptr, bc.ptr, ba.ptr], 3, 0, 1, 4096, 4096, 1, 4096, 0, 0, None,
                            _stream())
    torch.cuda.synchronize()
    assert st == 0
    want = [a.copy(), c.copy(), a.copy()]
    oracle.allreduce_inplace(want, root=0, dtype="f32", op="sum", rows=1, cols=4096, ld=4096,
                             valid_rows=1, valid_cols=4096)
    assert np.array_equal(ba.download("f32"), want[0])
    assert np.array_equal(bc.download("f32"), want[1])


def test_allreduce_full_size_workload():
    w = W.WORKLOADS["n16_i32_4096x4096"]
    srcs = W.make_sources(w)
    bufs = _upload(srcs, [0] * w.nranks)
    say("allreduce full n16_i32_4096x4096 sum")
    st = B.ptored_allreduce([b.ptr for b in bufs], w.nranks, 0, w.rows, w.cols, w.ld,
                            w.valid_rows, w.valid_cols, 3, 0, None, _stream())
    torch.cuda.synchronize()
    assert st == 0
    want = np.sum(np.stack([s.astype(np.int64) for s in srcs]), axis=0)
    want = ((want + 2**31) % 2**32 - 2**31).astype(np.int32)
    for b in bufs:
        assert np.array_equal(b.download("i32"), want)


# ------------------------------------------------------ ring reduce-scatter ---

# Launch variants of the reduce-scatter: (label, flags, blocks_per_cu,
# max_launch_bytes, misaligned dst 0).  The default takes one launch over
# every segment, the misaligned case included (its other streams are read
# and written unaligned); PTORED_SEGMENT_LAUNCHES takes one per segment.
RING_VARIANTS = [
    ("single", 0, 0, 0, False),
    ("elementwise", B.PTORED_FORCE_ELEMENTWISE, 0, 0, False),
    ("runtime_n", B.PTORED_FORCE_RUNTIME_N, 0, 0, False),
    ("per_segment", B.PTORED_SEGMENT_LAUNCHES, 0, 0, False),
    ("windows_1008", 0, 0, 1008, False),
    ("persistent", 0, 1, 0, False),
    ("misaligned", 0, 0, 0, True),
    ("windows_4096", B.PTORED_FORCE_RUNTIME_N, 0, 4096, False),
]


@pytest.mark.parametrize("dtype", DT)
def test_reduce_scatter_ring_random(dtype):
    rng = np.random.default_rng({"f32": 41, "bf16": 42, "f16": 43, "i32": 44}[dtype])
    for case in range(40):
        n = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 20, 64]))
        count = int(rng.choice([0, 1, 5, 20, 63, 100, 1000, 4099, 70001]))
        op = OPS[case % 4]
        label, flags, bpc, mlb, misaligned = RING_VARIANTS[case % len(RING_VARIANTS)]
        in_place = case % 3 == 0 and not misaligned
        srcs = [_rand_elems(dtype, rng, max(count, 1), wild=0.05) for _ in range(n)]
        sb = _upload(srcs, [0] * n)
        if in_place:
            db = sb
            d0 = [s.copy() for s in srcs]
        else:
            offs = [ESIZE[dtype] if (misaligned and s == 0) else 0 for s in range(n)]
            db = [DevBuf(max(count, 1) * ESIZE[dtype], o, fill=0xFF) for o in offs]
            d0 = [sentinel(dtype, max(count, 1)) for _ in range(n)]
        say(f"ring#{case} {dtype} {op} N={n} count={count} in_place={in_place} {label}")
        st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], n, [b.ptr for b in db], count,
                                          B.DTYPES[dtype], B.OPS[op],
                                          B.tuning(flags=flags, blocks_per_cu=bpc,
                                                   max_launch_bytes=mlb),
                                          _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = [d.copy() for d in d0]
        oracle.reduce_scatter_ring([s.copy() for s in srcs], want, count=count, dtype=dtype,
                                   op=op)
        for s in range(n):
            got = db[s].download(dtype)
            assert compare(dtype, got, want[s]).all(), (case, s)
            assert db[s].guards_intact()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_reduce_scatter_ring_ragged_segments(dtype):
    """Segment bounds off the 16-byte grid (f32: floor(i * count / N) with
    count not a multiple of 4N; bf16: the last segment short or empty), and
    windows whose edges fall inside segments, on the single-launch path."""
    rng = np.random.default_rng(47)
    for count, n, mlb in ((4099, 7, 0), (4099, 7, 528), (37, 5, 0), (17, 16, 0),
                          (33, 3, 16), (65537, 16, 8192), (250, 64, 0)):
        srcs = [_rand_elems(dtype, rng, count, wild=0.05) for _ in range(n)]
        sb = _upload(srcs, [0] * n)
        db = [DevBuf(count * ESIZE[dtype], 0, fill=0xFF) for _ in range(n)]
        say(f"ring ragged {dtype} count={count} N={n} mlb={mlb}")
        st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], n, [b.ptr for b in db], count,
                                          B.DTYPES[dtype], B.OPS["sum"],
                                          B.tuning(max_launch_bytes=mlb), _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = [sentinel(dtype, count) for _ in range(n)]
        oracle.reduce_scatter_ring([s.copy() for s in srcs], want, count=count, dtype=dtype,
                                   op="sum")
        for s in range(n):
            assert compare(dtype, db[s].download(dtype), want[s]).all(), (count, n, mlb, s)
            assert db[s].guards_intact()


def test_reduce_scatter_ring_full_size_bf16():
    w = W.WORKLOADS["n8_bf16_8192x8192"]
    srcs = W.make_sources(w)
    count = w.buffer_elems
    sb = _upload(srcs, [0] * w.nranks)
    say("ring full n8_bf16_8192x8192 sum in place")
    st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], w.nranks, [b.ptr for b in sb], count,
                                      1, 0, None, _stream())
    torch.cuda.synchronize()
    assert st == 0
    bounds = oracle.ring_bounds(count, w.nranks, "bf16")
    rng = np.random.default_rng(45)
    for s in range(w.nranks):
        got = sb[s].download("bf16")
        # sampled windows of each segment, computed by the oracle one by one
        for start in list(rng.integers(bounds[s], bounds[s + 1] - 4096, 3)) + [bounds[s],
                                                                               bounds[s + 1] - 4096]:
            lo, hi = int(start), int(start) + 4096
            sub = [np.ascontiguousarray(x[lo:hi]) for x in srcs]
            ring = [sub[(s + 1 + k) % w.nranks] for k in range(w.nranks)]
            want = sentinel("bf16", hi - lo)
            oracle.treduce(ring, want, root=0, dtype="bf16", op="sum", rows=1, cols=hi - lo,
                           ld=hi - lo, valid_rows=1, valid_cols=hi - lo)
            assert np.array_equal(got[lo:hi], want), (s, lo)
        # outside its own segment rank s's window is untouched
        outside = np.ones(count, bool)
        outside[bounds[s]:bounds[s + 1]] = False
        assert np.array_equal(got[outside], srcs[s][outside])


def test_reduce_scatter_ring_full_size_i32():
    """n16_i32_4096x4096 reduce-scatter into separate dsts: i32 sums wrap and
    are exact in any order, so every segment is checked whole against the
    wrapped sum; sampled windows against the oracle's ring-order fold."""
    w = W.WORKLOADS["n16_i32_4096x4096"]
    srcs = W.make_sources(w)
    count = w.buffer_elems
    sb = _upload(srcs, [0] * w.nranks)
    db = [DevBuf(count * 4, 0, fill=0xFF) for _ in range(w.nranks)]
    say("ring full n16_i32_4096x4096 sum")
    st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], w.nranks, [b.ptr for b in db], count,
                                      B.DTYPES["i32"], B.OPS["sum"], None, _stream())
    torch.cuda.synchronize()
    assert st == 0
    bounds = oracle.ring_bounds(count, w.nranks, "i32")
    total = np.zeros(count, np.int64)
    for x in srcs:
        total += x
    total = total.astype(np.uint32).view(np.int32)  # wrap to 32 bits
    rng = np.random.default_rng(46)
    for s in range(w.nranks):
        got = db[s].download("i32")
        lo, hi = int(bounds[s]), int(bounds[s + 1])
        assert np.array_equal(got[lo:hi], total[lo:hi]), s
        assert np.all(got[:lo].view(np.uint32) == 0xFFFFFFFF)
        assert np.all(got[hi:].view(np.uint32) == 0xFFFFFFFF)
        a = int(rng.integers(lo, hi - 1024))
        sub = [np.ascontiguousarray(x[a:a + 1024]) for x in srcs]
        ring = [sub[(s + 1 + k) % w.nranks] for k in range(w.nranks)]
        want = sentinel("i32", 1024)
        oracle.treduce(ring, want, root=0, dtype="i32", op="sum", rows=1, cols=1024, ld=1024,
                       valid_rows=1, valid_cols=1024)
        assert np.array_equal(got[a:a + 1024], want), (s, a)


# ------------------------------------------------------------ push-with-add ---

UNIT = {"f32": 2.0 ** -24, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def _finite_values(dtype, rng, n):
    v = (rng.standard_normal(n) * np.exp2(rng.integers(-4, 4, n))).astype(np.float32)
    if dtype == "f32":
        return v
    if dtype == "i32":
        return rng.integers(-2**30, 2**30, n, dtype=np.int64).astype(np.int32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", DT)
def test_accumulate_add_random(dtype):
    rng = np.random.default_rng({"f32": 51, "bf16": 52, "f16": 53, "i32": 54}[dtype])
    es = ESIZE[dtype]
    for case in range(16):
        n = int(rng.choice([1, 2, 3, 8, 16, 33]))
        rows = int(rng.integers(1, 30))
        cols = int(rng.integers(1, 700))
        ld = cols + int(rng.choice([0, 1, 8]))
        vr, vc = int(rng.integers(1, rows + 1)), int(rng.integers(1, cols + 1))
        flags = [0, B.PTORED_FORCE_ELEMENTWISE, B.PTORED_FORCE_ROWS][case % 3] | (
            B.PTORED_ACC_PER_RANK if case % 2 else 0)
        size = (rows - 1) * ld + cols
        srcs = [_finite_values(dtype, rng, size) for _ in range(n)]
        d0 = _finite_values(dtype, rng, size)
        sb = _upload(srcs, [0 if case % 2 else int(rng.integers(0, 4)) * es for _ in range(n)])
        db = _upload([d0], [0 if case % 4 else 2 * es])[0]
        say(f"accumulate#{case} {dtype} N={n} {rows}x{cols} ld={ld} valid={vr}x{vc} "
            f"flags={flags}")
        st = B.ptored_accumulate_add([b.ptr for b in sb], n, db.ptr, rows, cols, ld, vr, vc,
                                     B.DTYPES[dtype], B.tuning(flags=flags), _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        got = db.download(dtype)
        want = d0.copy()
        exact, absum = oracle.accumulate_add(srcs, want, dtype=dtype, rows=rows, cols=cols,
                                             ld=ld, valid_rows=vr, valid_cols=vc)
        m = valid_mask(rows, ld, vr, vc, size)
        assert np.array_equal(got[~m].view(np.uint8), d0[~m].view(np.uint8)), case
        assert db.guards_intact()
        if dtype == "i32":
            # wrap-around integer sums have one possible result
            assert compare(dtype, got[m], want[m]).all(), case
        else:
            g = oracle.to_double(dtype, bits(dtype, got[m]).astype(np.uint32))
            bound = n * UNIT[dtype] * absum * 1.0001
            assert np.all(np.abs(g - exact) <= bound), case


@pytest.mark.parametrize("dtype", DT)
def test_accumulate_in_one_call_via_treduce(dtype):
    """dst += src_0 + ... + src_{N-1} in rank order, in one reduction call: dst
    as the root source and the destination (exact alias).  Bit-exact against
    the oracle's rank-order accumulation."""
    rng = np.random.default_rng({"f32": 81, "bf16": 82, "f16": 83, "i32": 84}[dtype])
    for case in range(6):
        n = int(rng.choice([1, 3, 8, 15]))
        rows, cols = int(rng.integers(1, 40)), int(rng.integers(1, 600))
        ld = cols + int(rng.choice([0, 5, 8]))
        vr, vc = int(rng.integers(1, rows + 1)), int(rng.integers(1, cols + 1))
        size = (rows - 1) * ld + cols
        srcs = [_rand_elems(dtype, rng, size, wild=0.05) for _ in range(n)]
        d0 = _rand_elems(dtype, rng, size, wild=0.05)
        bufs = _upload([d0] + srcs, [0] * (n + 1))
        say(f"accumulate via treduce#{case} {dtype} N={n} {rows}x{cols} ld={ld} valid={vr}x{vc}")
        st = B.ptored_treduce([b.ptr for b in bufs], n + 1, 0, bufs[0].ptr, rows, cols, ld, vr,
                              vc, B.DTYPES[dtype], B.OPS["sum"], _stream())
        torch.cuda.synchronize()
        assert st == 0, B.ptored_status_string(st)
        want = d0.copy()
        oracle.accumulate_add(srcs, want, dtype=dtype, rows=rows, cols=cols, ld=ld,
                              valid_rows=vr, valid_cols=vc)
        assert compare(dtype, bufs[0].download(dtype), want).all(), case


def test_accumulate_add_full_size_i32_exact():
    w = W.WORKLOADS["n16_i32_4096x4096"]
    srcs = W.make_sources(w)
    sb = _upload(srcs, [0] * w.nranks)
    d0 = np.arange(w.buffer_elems, dtype=np.int32)
    db = _upload([d0], [0])[0]
    say("accumulate full n16_i32_4096x4096")
    st = B.ptored_accumulate_add([b.ptr for b in sb], w.nranks, db.ptr, w.rows, w.cols, w.ld,
                                 w.valid_rows, w.valid_cols, 3, None, _stream())
    torch.cuda.synchronize()
    assert st == 0
    want = d0.astype(np.int64) + np.sum(np.stack([s.astype(np.int64) for s in srcs]), axis=0)
    want = ((want + 2**31) % 2**32 - 2**31).astype(np.int32)
    assert np.array_equal(db.download("i32"), want)


# ------------------------------------------------------------ tensor wrappers ---

def test_tensor_wrappers_of_the_collectives():
    """allreduce / reduce_scatter_ring / accumulate_add / ring_bounds on torch
    tensors (2-D views with a pitch, a side stream) against the oracle."""
    import cross_rank_collective_amd as crc

    rng = np.random.default_rng(97)
    n, rows, cols, ld = 5, 37, 300, 304
    host = [rng.standard_normal((rows, ld)).astype(np.float32) for _ in range(n)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bufs = [torch.from_numpy(h).cuda()[:, :cols] for h in host]   # 2-D views, ld 304
        crc.allreduce(bufs, op="max", root=2, valid=(rows - 1, cols - 3))
    s.synchronize()
    want = [h.reshape(-1).copy() for h in host]
    oracle.allreduce_inplace(want, root=2, dtype="f32", op="max", rows=rows, cols=ld, ld=ld,
                             valid_rows=rows - 1, valid_cols=cols - 3)
    for b, w_ in zip(bufs, want):
        got = b.cpu().numpy()
        assert np.array_equal(got, w_.reshape(rows, ld)[:, :cols])

    count = 10007
    srcs = [torch.from_numpy(rng.integers(-2 ** 20, 2 ** 20, count, dtype=np.int32)).cuda()
            for _ in range(n)]
    dsts = [torch.full((count,), -1, dtype=torch.int32, device="cuda") for _ in range(n)]
    crc.reduce_scatter_ring(srcs, dsts, op="sum")
    torch.cuda.synchronize()
    want = [sentinel("i32", count) for _ in range(n)]
    oracle.reduce_scatter_ring([t.cpu().numpy() for t in srcs], want, count=count, dtype="i32",
                               op="sum")
    for d, w_ in zip(dsts, want):
        assert np.array_equal(d.cpu().numpy(), w_)

    # empty tensors (no storage): nothing to reduce, no error, nothing launched
    e = [torch.empty(0, 8, device="cuda") for _ in range(3)]
    crc.treduce(e[:2], e[2])
    crc.allreduce(e)
    crc.accumulate_add(e[:2], e[2])
    crc.reduce_scatter_ring([torch.empty(0, device="cuda")] * 2,
                            [torch.empty(0, device="cuda")] * 2)
    # a zero-width valid rectangle on real tensors writes nothing
    a = torch.ones(4, 8, device="cuda")
    d = torch.full((4, 8), 7.0, device="cuda")
    crc.treduce([a, a], d, valid=(4, 0))
    torch.cuda.synchronize()
    assert bool((d == 7.0).all())
    assert crc.ring_bounds(count, n, torch.int32) == list(oracle.ring_bounds(count, n, "i32"))

    srcs = [torch.from_numpy(rng.integers(-2 ** 20, 2 ** 20, (rows, cols), dtype=np.int32))
            .cuda() for _ in range(n)]
    d0 = rng.integers(-2 ** 20, 2 ** 20, (rows, cols), dtype=np.int32)
    dst = torch.from_numpy(d0).cuda()
    crc.accumulate_add(srcs, dst, valid=(rows, cols - 1))
    torch.cuda.synchronize()
    want = d0.reshape(-1).copy()
    oracle.accumulate_add([t.cpu().numpy().reshape(-1) for t in srcs], want, dtype="i32",
                          rows=rows, cols=cols, ld=cols, valid_rows=rows, valid_cols=cols - 1)
    assert np.array_equal(dst.cpu().numpy().reshape(-1), want)
    with pytest.raises(crc.PtoredError):
        crc.accumulate_add(srcs, srcs[0])  # dst may not be a source
