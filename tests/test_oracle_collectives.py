"""Pins for the oracle's collective variants (CPU): the ring segment schedule
and its reduce-scatter share, the in-place allreduce store-back, and the
push-with-add accumulation."""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import brute
from tests.test_oracle_pins import (_bits, _from_values, _isnan_bits, _random_bits, _sentinel,
                                    _to_brute, _values)

DT = ["f32", "bf16", "f16", "i32"]


def _golden_bounds():
    path = os.path.join(os.path.dirname(__file__), "golden", "ring_segment_bounds.txt")
    out = []
    for line in open(path):
        f = line.split("#")[0].split()
        if f:
            out.append((f[0], int(f[1]), int(f[2]), [int(x) for x in f[3:]]))
    return out


@pytest.mark.parametrize("case", _golden_bounds())
def test_ring_bounds_worked_examples(case):
    dtype, size, nr, want = case
    assert list(oracle.ring_bounds(size, nr, dtype)) == want


def test_ring_bounds_properties():
    rng = np.random.default_rng(3)
    for _ in range(300):
        size = int(rng.integers(0, 5000))
        nr = int(rng.integers(1, 65))
        for dtype in DT:
            b = oracle.ring_bounds(size, nr, dtype)
            assert b[0] == 0 and b[-1] == size
            assert np.all(np.diff(b) >= 0)
            if dtype in ("f16", "bf16"):
                assert all(x % 16 == 0 or x == size for x in b[1:-1])
            else:  # balanced: segment lengths differ by at most one
                d = np.diff(b)
                assert d.max() - d.min() <= 1


def test_reduce_scatter_ring_fold_order():
    """Segment s folds ranks s+1, s+2, ..., s (mod N).  With (1, 1e8, -1e8)
    held by ranks (0, 1, 2) in binary32: segment 0 folds 1e8 + -1e8 + 1 = 1;
    segment 1 folds -1e8 + 1 + 1e8 = 0 (1 is absorbed); segment 2 folds
    1 + 1e8 + -1e8 = 0."""
    n = 48  # three f32 segments of 16 elements
    vals = (1.0, 1e8, -1e8)
    srcs = [np.full(n, v, np.float32) for v in vals]
    dsts = [_sentinel("f32", n) for _ in range(3)]
    oracle.reduce_scatter_ring(srcs, dsts, count=n, dtype="f32", op="sum")
    b = oracle.ring_bounds(n, 3, "f32")
    assert list(b) == [0, 16, 32, 48]
    assert np.all(dsts[0][0:16] == 1.0)
    assert np.all(dsts[1][16:32] == 0.0)
    assert np.all(dsts[2][32:48] == 0.0)
    # outside its own segment every dst is untouched
    assert np.all(dsts[0][16:].view(np.int32) == -1)
    assert np.all(dsts[1][:16].view(np.int32) == -1) and np.all(dsts[1][32:].view(np.int32) == -1)


@pytest.mark.parametrize("dtype", DT)
def test_reduce_scatter_ring_brute_force(dtype):
    rng = np.random.default_rng({"f32": 5, "bf16": 6, "f16": 7, "i32": 8}[dtype])
    for case in range(12):
        n = int(rng.choice([1, 2, 3, 5, 8]))
        count = int(rng.integers(0, 70))
        op = ["sum", "max", "min", "prod"][case % 4]
        srcs = [_random_bits(dtype, rng, max(count, 1)) for _ in range(n)]
        dsts = [_sentinel(dtype, max(count, 1)) for _ in range(n)]
        oracle.reduce_scatter_ring(srcs, dsts, count=count, dtype=dtype, op=op)
        b = oracle.ring_bounds(count, n, dtype)
        bs = [_to_brute(dtype, s) for s in srcs]
        for s in range(n):
            got = _bits(dtype, dsts[s])
            for j in range(max(count, 1)):
                if b[s] <= j < b[s + 1]:
                    acc = bs[(s + 1) % n][j]
                    for k in range(2, n + 1):
                        acc = brute.combine(dtype, op, acc, bs[(s + k) % n][j])
                    if dtype == "i32":
                        assert int(dsts[s][j]) == acc
                    elif acc == -1:
                        assert _isnan_bits(dtype, [got[j]])[0]
                    else:
                        assert int(got[j]) == acc, (case, s, j)
                else:
                    assert got[j] == _bits(dtype, _sentinel(dtype, 1))[0]


@pytest.mark.parametrize("dtype", DT)
def test_reduce_scatter_ring_closed_forms(dtype):
    for n in (1, 2, 5, 16):
        count = 333
        ones = [_from_values(dtype, np.ones(count)) for _ in range(n)]
        ids = [_from_values(dtype, np.full(count, r)) for r in range(n)]
        for srcs, op, want in ((ones, "sum", n), (ids, "sum", n * (n - 1) // 2),
                               (ids, "max", n - 1), (ids, "min", 0)):
            dsts = [_sentinel(dtype, count) for _ in range(n)]
            oracle.reduce_scatter_ring(srcs, dsts, count=count, dtype=dtype, op=op)
            b = oracle.ring_bounds(count, n, dtype)
            for s in range(n):
                assert np.all(_values(dtype, dsts[s][b[s]:b[s + 1]]) == want)


@pytest.mark.parametrize("dtype", DT)
def test_accumulate_add_rank_order_and_exact_sum(dtype):
    """dst + src_0 + ... in rank order, each step in the element type; and the
    exact sum, against the brute force (Fractions for the exact value)."""
    rng = np.random.default_rng({"f32": 15, "bf16": 16, "f16": 17, "i32": 18}[dtype])
    rows, cols, ld, vr, vc, n = 4, 9, 11, 3, 7, 5
    size = (rows - 1) * ld + cols
    srcs = [_random_bits(dtype, rng, size) for _ in range(n)]
    dst0 = _random_bits(dtype, rng, size)
    dst = dst0.copy()
    exact, absum = oracle.accumulate_add(srcs, dst, dtype=dtype, rows=rows, cols=cols, ld=ld,
                                         valid_rows=vr, valid_cols=vc)
    got = _bits(dtype, dst)
    bd, bs = _to_brute(dtype, dst0), [_to_brute(dtype, s) for s in srcs]
    k = 0
    for i in range(vr):
        for j in range(vc):
            idx = i * ld + j
            acc = bd[idx]
            for r in range(n):
                acc = brute.combine(dtype, "sum", acc, bs[r][idx])
            if dtype == "i32":
                assert int(dst[idx]) == acc
            elif acc == -1:
                assert _isnan_bits(dtype, [got[idx]])[0]
            else:
                assert int(got[idx]) == acc
                terms = [brute._value(dtype, bd[idx])] + [brute._value(dtype, x[idx]) for x in bs]
                if all(np.isfinite(terms)):
                    ex = sum(Fraction(t) for t in terms)
                    assert abs(Fraction(exact[k]) - ex) <= Fraction(absum[k]) * 2 ** -50
            k += 1
    # outside the valid rectangle dst is unchanged
    m = np.zeros((rows, ld), bool)
    m[:vr, :vc] = True
    m = m.reshape(-1)[:size]
    assert np.array_equal(_bits(dtype, dst)[~m], _bits(dtype, dst0)[~m])


def test_accumulate_add_closed_form():
    srcs = [np.ones(64, np.float32)] * 7
    dst = np.full(64, 2.0, np.float32)
    oracle.accumulate_add(srcs, dst, dtype="f32", rows=8, cols=8, ld=8, valid_rows=8,
                          valid_cols=8)
    assert np.all(dst == 9.0)
    d = np.full(64, 2**31 - 1, np.int32)
    oracle.accumulate_add([np.ones(64, np.int32)] * 2, d, dtype="i32", rows=1, cols=64, ld=64,
                          valid_rows=1, valid_cols=64)
    assert np.all(d == -2**31 + 1)  # wraps


@pytest.mark.parametrize("dtype", DT)
def test_allreduce_inplace_matches_treduce_into_every_buffer(dtype):
    rng = np.random.default_rng(21)
    rows, cols, ld, vr, vc, n = 5, 12, 13, 4, 11, 6
    size = (rows - 1) * ld + cols
    for op in ("sum", "max", "min", "prod"):
        bufs = [_random_bits(dtype, rng, size) for _ in range(n)]
        before = [b.copy() for b in bufs]
        want = _sentinel(dtype, size)
        oracle.treduce(before, want, root=2, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                       valid_rows=vr, valid_cols=vc)
        oracle.allreduce_inplace(bufs, root=2, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                                 valid_rows=vr, valid_cols=vc)
        m = np.zeros((rows, ld), bool)
        m[:vr, :vc] = True
        m = m.reshape(-1)[:size]
        for b, b0 in zip(bufs, before):
            assert np.array_equal(_bits(dtype, b)[m], _bits(dtype, want)[m])
            assert np.array_equal(_bits(dtype, b)[~m], _bits(dtype, b0)[~m])
