"""A seeded sweep over the whole launch space: every entry point with shapes,
rank counts, roots, buffer offsets (aligned, one shared lead, each its own),
in-place aliasing, forcing flags, grid policies and launch windows drawn
together, each call checked against the oracle.

Bar as in the parity tests: bit-exact (NaN by NaN-ness) for the reduction,
the allreduce and the reduce-scatter, exact for i32 push-with-add and within
the rounding of N additions in any order for float push-with-add; cells
outside the valid rectangle, guard bands and sources untouched.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from tests.gpu_helpers import DevBuf, ESIZE, compare, run_gpu, say, sentinel, valid_mask
from tests.test_parity_gpu import _check, _rand_elems

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "max", "min", "prod"]
RANKS = [1, 2, 2, 3, 4, 5, 6, 7, 8, 8, 11, 16, 16, 17, 24, 64]
FLAG_SETS = [0, 0, 0, B.PTORED_FORCE_ELEMENTWISE, B.PTORED_FORCE_ROWS,
             B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK,
             B.PTORED_FORCE_RUNTIME_N, B.PTORED_LDS_PINGPONG, B.PTORED_FULL_OCCUPANCY,
             B.PTORED_FORCE_RUNTIME_N | B.PTORED_FULL_OCCUPANCY,
             B.PTORED_LDS_PINGPONG | B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK]
MAX_ELEMS = 40000  # per buffer
# PTORED_SWEEP_SCALE=k draws k times as many calls per test (default 1).
SCALE = max(1, int(os.environ.get("PTORED_SWEEP_SCALE", "1")))


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _shape(rng, es):
    """rows, cols, ld, valid_rows, valid_cols with at most MAX_ELEMS elements."""
    kind = rng.integers(0, 3)
    step = 16 // es  # elements per 16 bytes
    pitch16 = rng.random() < 0.7  # the vector path needs 16-byte row pitches
    if kind == 0:  # one long row
        cols = int(rng.integers(1, MAX_ELEMS))
        rows, ld = 1, cols
    elif kind == 1:  # rows back to back (contiguous when fully valid)
        cols = int(rng.integers(1, 2000))
        if pitch16:
            cols = (cols + step - 1) // step * step
        rows = int(rng.integers(1, max(2, MAX_ELEMS // cols)))
        ld = cols
    else:  # pitched rows
        cols = int(rng.integers(1, 3000))
        ld = cols + int(rng.choice([1, 2, 3, 5, 8, 16, 64]))
        if pitch16:
            ld = (ld + step - 1) // step * step
        rows = int(rng.integers(1, max(2, MAX_ELEMS // ld)))
    vr = rows if rng.random() < 0.4 else int(rng.integers(1, rows + 1))
    vc = cols if rng.random() < 0.4 else int(rng.integers(1, cols + 1))
    if rng.random() < 0.03:
        vr, vc = (0, vc) if rng.random() < 0.5 else (vr, 0)
    return rows, cols, ld, vr, vc


def _offsets(rng, es, n):
    """Byte offsets of n buffers (+ one more for a dst): on the 16-byte grid,
    one shared offset within a 16-byte block, one shared offset within
    1 KiB, or each its own."""
    kind = rng.choice([0, 0, 1, 1, 2, 2, 3])
    if kind == 0:
        return [16 * int(rng.integers(0, 8)) for _ in range(n + 1)]
    if kind == 1:
        lead = int(rng.choice(list(range(es, 16, es))))
        return [lead + 16 * int(rng.integers(0, 8)) for _ in range(n + 1)]
    if kind == 2:
        return [es * int(rng.integers(0, 1024 // es))] * (n + 1)
    return [es * int(rng.integers(0, 32)) for _ in range(n + 1)]


def _tuning(rng, total_bytes):
    flags = int(rng.choice(FLAG_SETS))
    bpc = int(rng.choice([0, 0, 0, 0, 0, 1, 2, -1]))
    if rng.random() < 0.3:  # small launch windows, at most ~500 launches per call
        lo = max(16, total_bytes // 500)
        mlb = int(rng.integers(lo, max(lo + 1, total_bytes + 1)))
    else:
        mlb = 0
    return B.tuning(flags=flags, blocks_per_cu=bpc, max_launch_bytes=mlb)


def _tstr(t):
    return f"flags={t.flags:#x} bpc={t.blocks_per_cu} mlb={t.max_launch_bytes}"


@pytest.mark.parametrize("chunk", range(8))
def test_sweep_treduce(chunk):
    rng = np.random.default_rng(9100 + chunk)
    for case in range(100 * SCALE):
        dtype = DT[int(rng.integers(0, 4))]
        op = OPS[int(rng.integers(0, 4))]
        es = ESIZE[dtype]
        n = int(rng.choice(RANKS))
        root = int(rng.integers(0, n))
        rows, cols, ld, vr, vc = _shape(rng, es)
        offs = _offsets(rng, es, n)
        size = (rows - 1) * ld + cols
        t = _tuning(rng, size * es)
        alias = int(rng.integers(0, n)) if rng.random() < 0.12 else -1
        srcs = [_rand_elems(dtype, rng, size, wild=0.05) for _ in range(n)]
        label = (f"sweep{chunk}#{case} treduce {dtype} {op} N={n} root={root} "
                 f"{rows}x{cols} ld={ld} valid={vr}x{vc} offs={offs[:3]} alias={alias} "
                 f"{_tstr(t)}")
        dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc,
                                offsets=offs[:n], dst_offset=offs[n], tuning=t, alias=alias,
                                label=label)
        assert st == 0, (label, B.ptored_status_string(st))
        _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, alias=alias,
               label=label)


def _upload(arrs, offs, fill=0xA5):
    out = []
    for a, o in zip(arrs, offs):
        b = DevBuf(a.size * a.itemsize, o, fill=fill)
        b.upload(a)
        out.append(b)
    return out


def test_sweep_allreduce():
    rng = np.random.default_rng(9200)
    for case in range(200 * SCALE):
        dtype = DT[int(rng.integers(0, 4))]
        op = OPS[int(rng.integers(0, 4))]
        es = ESIZE[dtype]
        n = int(rng.choice(RANKS))
        root = int(rng.integers(0, n))
        rows, cols, ld, vr, vc = _shape(rng, es)
        offs = _offsets(rng, es, n)
        size = (rows - 1) * ld + cols
        t = _tuning(rng, size * es)
        srcs = [_rand_elems(dtype, rng, size, wild=0.05) for _ in range(n)]
        bufs = _upload(srcs, offs[:n])
        label = (f"sweep allreduce#{case} {dtype} {op} N={n} root={root} {rows}x{cols} ld={ld} "
                 f"valid={vr}x{vc} offs={offs[:3]} {_tstr(t)}")
        say(label)
        st = B.ptored_allreduce([b.ptr for b in bufs], n, root, rows, cols, ld, vr, vc,
                                B.DTYPES[dtype], B.OPS[op], t, _stream())
        torch.cuda.synchronize()
        assert st == 0, (label, B.ptored_status_string(st))
        want = [s.copy() for s in srcs]
        oracle.allreduce_inplace(want, root=root, dtype=dtype, op=op, rows=rows, cols=cols,
                                 ld=ld, valid_rows=vr, valid_cols=vc)
        m = valid_mask(rows, ld, vr, vc, size)
        for r, b in enumerate(bufs):
            got = b.download(dtype)
            assert compare(dtype, got[m], want[r][m]).all(), (label, r)
            assert np.array_equal(got[~m].view(np.uint8), srcs[r][~m].view(np.uint8)), (label, r)
            assert b.guards_intact(), (label, r)


def test_sweep_reduce_scatter_ring():
    rng = np.random.default_rng(9300)
    for case in range(200 * SCALE):
        dtype = DT[int(rng.integers(0, 4))]
        op = OPS[int(rng.integers(0, 4))]
        es = ESIZE[dtype]
        n = int(rng.choice(RANKS))
        count = int(rng.choice([0, 1, int(rng.integers(2, 200)), int(rng.integers(200, 5000)),
                                int(rng.integers(5000, MAX_ELEMS))]))
        offs = _offsets(rng, es, 2 * n)
        t = _tuning(rng, count * es)
        if rng.random() < 0.3:
            t.flags |= B.PTORED_SEGMENT_LAUNCHES
        in_place = rng.random() < 0.3
        srcs = [_rand_elems(dtype, rng, max(count, 1), wild=0.05) for _ in range(n)]
        sb = _upload(srcs, offs[:n])
        if in_place:
            db, d0 = sb, [s.copy() for s in srcs]
        else:
            db = [DevBuf(max(count, 1) * es, o, fill=0xFF) for o in offs[n:2 * n]]
            d0 = [sentinel(dtype, max(count, 1)) for _ in range(n)]
        label = (f"sweep ring#{case} {dtype} {op} N={n} count={count} in_place={in_place} "
                 f"offs={offs[:3]} {_tstr(t)}")
        say(label)
        st = B.ptored_reduce_scatter_ring([b.ptr for b in sb], n, [b.ptr for b in db], count,
                                          B.DTYPES[dtype], B.OPS[op], t, _stream())
        torch.cuda.synchronize()
        assert st == 0, (label, B.ptored_status_string(st))
        want = [d.copy() for d in d0]
        oracle.reduce_scatter_ring([s.copy() for s in srcs], want, count=count, dtype=dtype,
                                   op=op)
        for s in range(n):
            assert compare(dtype, db[s].download(dtype), want[s]).all(), (label, s)
            assert db[s].guards_intact(), (label, s)
        if not in_place:
            for s in range(n):
                assert np.array_equal(sb[s].download(dtype).view(np.uint8),
                                      srcs[s].view(np.uint8)), (label, "src", s)


def test_sweep_accumulate_i32():
    """i32 push-with-add: wrapping sums are the same in any order, so exact."""
    rng = np.random.default_rng(9400)
    for case in range(100 * SCALE):
        n = int(rng.choice(RANKS))
        rows, cols, ld, vr, vc = _shape(rng, 4)
        offs = _offsets(rng, 4, n)
        size = (rows - 1) * ld + cols
        t = _tuning(rng, size * 4)
        t.blocks_per_cu = 0
        if case % 2:
            t.flags |= B.PTORED_ACC_PER_RANK
        srcs = [_rand_elems("i32", rng, size) for _ in range(n)]
        d0 = _rand_elems("i32", rng, size)
        sb = _upload(srcs, offs[:n])
        dd = _upload([d0], [offs[n]])[0]
        label = (f"sweep accumulate#{case} i32 N={n} {rows}x{cols} ld={ld} valid={vr}x{vc} "
                 f"offs={offs[:3]} {_tstr(t)}")
        say(label)
        st = B.ptored_accumulate_add([b.ptr for b in sb], n, dd.ptr, rows, cols, ld, vr, vc,
                                     B.DTYPES["i32"], t, _stream())
        torch.cuda.synchronize()
        assert st == 0, (label, B.ptored_status_string(st))
        want = d0.copy()
        oracle.accumulate_add(srcs, want, dtype="i32", rows=rows, cols=cols, ld=ld,
                              valid_rows=vr, valid_cols=vc)
        assert np.array_equal(dd.download("i32"), want), label
        assert dd.guards_intact(), label


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_sweep_accumulate_float(dtype):
    """Float push-with-add.  Folded first (the default): dst + fold(srcs) bit
    for bit.  Per rank: the additions land in any order, so each valid
    element must lie within the rounding of N additions of the exact sum.
    Everything outside the valid rectangle keeps its bits."""
    from tests.gpu_helpers import bits
    from tests.test_collectives_gpu import UNIT, _finite_values
    from tests.test_push_gpu import _fold_then_add
    rng = np.random.default_rng({"f32": 9501, "bf16": 9502, "f16": 9503}[dtype])
    es = ESIZE[dtype]
    for case in range(40 * SCALE):
        n = int(rng.choice(RANKS))
        rows, cols, ld, vr, vc = _shape(rng, es)
        offs = _offsets(rng, es, n)
        size = (rows - 1) * ld + cols
        t = _tuning(rng, size * es)
        t.blocks_per_cu = 0
        per_rank = case % 2 == 1
        if per_rank:
            t.flags |= B.PTORED_ACC_PER_RANK
        srcs = [_finite_values(dtype, rng, size) for _ in range(n)]
        d0 = _finite_values(dtype, rng, size)
        sb = _upload(srcs, offs[:n])
        dd = _upload([d0], [offs[n]])[0]
        label = (f"sweep accumulate#{case} {dtype} N={n} {rows}x{cols} ld={ld} valid={vr}x{vc} "
                 f"offs={offs[:3]} dst_off={offs[n]} {_tstr(t)}")
        say(label)
        st = B.ptored_accumulate_add([b.ptr for b in sb], n, dd.ptr, rows, cols, ld, vr, vc,
                                     B.DTYPES[dtype], t, _stream())
        torch.cuda.synchronize()
        assert st == 0, (label, B.ptored_status_string(st))
        got = dd.download(dtype)
        want = d0.copy()
        exact, absum = oracle.accumulate_add(srcs, want, dtype=dtype, rows=rows, cols=cols,
                                             ld=ld, valid_rows=vr, valid_cols=vc)
        m = valid_mask(rows, ld, vr, vc, size)
        assert np.array_equal(got[~m].view(np.uint8), d0[~m].view(np.uint8)), label
        assert dd.guards_intact(), label
        g = oracle.to_double(dtype, bits(dtype, got[m]).astype(np.uint32))
        bound = n * UNIT[dtype] * absum * 1.0001
        assert np.all(np.abs(g - exact) <= bound), label
        if not per_rank:
            folded, _ = _fold_then_add(srcs, d0, dtype, rows, cols, ld, vr, vc)
            assert compare(dtype, got, folded).all(), label
