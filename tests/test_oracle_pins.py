"""Pins for the CPU oracle (runs without a GPU).

Each test ties the oracle to something other than itself: library routines
(numpy / torch conversions and arithmetic), an independent brute force
(tests/brute.py), closed forms and invariants.  The cases are chosen so a
plausible slip in the oracle -- a dropped rank, a wrong order, a transposed
index, a wrong rounding threshold, a sign slip in Max/Min -- fails one of them.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from tests import brute

# NaN bit patterns and doubles beyond a format's range are cast on purpose.
pytestmark = pytest.mark.filterwarnings(
    "ignore:invalid value encountered in cast:RuntimeWarning",
    "ignore:overflow encountered in cast:RuntimeWarning")

DT = ["f32", "bf16", "f16", "i32"]
FLOAT_DT = ["f32", "bf16", "f16"]
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "i32": np.int32}


# ---------------------------------------------------------------- helpers ---

def _from_values(dtype, vals):
    """Element buffer holding the given real values (exactly representable)."""
    v = np.asarray(vals, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "i32":
        return v.astype(np.int32)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _values(dtype, buf):
    if dtype == "f32":
        return buf.astype(np.float64)
    if dtype == "i32":
        return buf.astype(np.float64)
    if dtype == "f16":
        return buf.view(np.float16).astype(np.float64)
    return (buf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bits(dtype, buf):
    if dtype in ("f32", "i32"):
        return buf.view(np.uint32).astype(np.uint64)
    return buf.astype(np.uint64)


def _run(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst=None):
    if dst is None:
        dst = _sentinel(dtype, max(1, rows * ld))
    oracle.treduce(srcs, dst, root=root, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                   valid_rows=vr, valid_cols=vc)
    return dst


def _sentinel(dtype, n):
    if dtype == "f32":
        return np.full(n, -1, np.int32).view(np.float32)
    if dtype == "i32":
        return np.full(n, -1, np.int32)
    return np.full(n, 0xFFFF, np.uint16)


def _valid_mask(rows, ld, vr, vc):
    m = np.zeros((rows, ld), dtype=bool)
    m[:vr, :vc] = True
    return m.reshape(-1)


def _isnan_bits(dtype, bits):
    bits = np.asarray(bits, dtype=np.uint64)
    if dtype == "f32":
        return ((bits >> 23) & 0xFF == 0xFF) & (bits & 0x7FFFFF != 0)
    if dtype == "f16":
        return ((bits >> 10) & 0x1F == 0x1F) & (bits & 0x3FF != 0)
    return ((bits >> 7) & 0xFF == 0xFF) & (bits & 0x7F != 0)


def _same_bits(dtype, a, b):
    """Bitwise equality, NaN compared by NaN-ness only (float types)."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    if dtype == "i32":
        return a == b
    na, nb = _isnan_bits(dtype, a), _isnan_bits(dtype, b)
    return np.where(na | nb, na & nb, a == b)


# ------------------------------------------------ element formats (decode) ---

def test_decode_f16_every_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.to_double("f16", bits)
    want = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_decode_bf16_every_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    got = oracle.to_double("bf16", bits)
    # bfloat16 is the upper half of a binary32 word
    want = (bits << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


# ---------------------------------------------- element formats (rounding) ---

def _hard_doubles(dtype, rng):
    """Doubles concentrated where rounding is delicate for `dtype`."""
    allb = np.arange(65536, dtype=np.uint32)
    if dtype == "f16":
        vals = allb.astype(np.uint16).view(np.float16).astype(np.float64)
    elif dtype == "bf16":
        vals = (allb << 16).view(np.float32).astype(np.float64)
    else:
        vals = rng.standard_normal(200000).astype(np.float32).astype(np.float64)
        vals = np.concatenate([vals, (rng.integers(0, 2**32, 200000, dtype=np.uint64)
                                      .astype(np.uint32).view(np.float32).astype(np.float64))])
    fin = np.sort(np.unique(vals[np.isfinite(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2.0  # exact in double for all three formats
    up = np.nextafter(mids, np.inf)
    dn = np.nextafter(mids, -np.inf)
    rand = np.exp2(rng.uniform(-160, 130, 100000)) * rng.choice([-1.0, 1.0], 100000)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 65536.0,
                        -65520.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26, 2.0**-133, 2.0**-134,
                        3.3895313892515355e38, 3.4e38, 1e300, -1e300, 2.0**-150, 2.0**-149])
    return np.concatenate([fin, mids, up, dn, rand, special])


def test_round_f16_matches_numpy():
    rng = np.random.default_rng(11)
    x = _hard_doubles("f16", rng)
    got = oracle.round_from_double("f16", x)
    want = x.astype(np.float16).view(np.uint16).astype(np.uint32)
    assert np.array_equal(got, want)


def test_round_f32_matches_numpy():
    rng = np.random.default_rng(12)
    x = _hard_doubles("f32", rng)
    got = oracle.round_from_double("f32", x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def test_round_bf16_matches_enumeration():
    """bf16 rounding against nearest-value search over every bf16 value."""
    rng = np.random.default_rng(13)
    x = _hard_doubles("bf16", rng)
    pick = rng.choice(x.size, 6000, replace=False)
    sample = np.concatenate([x[pick], _hard_doubles("bf16", rng)[-20:]])
    got = oracle.round_from_double("bf16", sample)
    f = brute.fmt("bf16")
    from fractions import Fraction
    for v, g in zip(sample, got):
        if np.isinf(v):
            want = f.round(float(v))
        else:
            want = f.round(Fraction(float(v)), negative_zero=bool(np.signbit(v)))
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_round_bf16_matches_torch_on_f32_inputs():
    """For binary32 inputs torch's float->bf16 conversion is a single RNE."""
    rng = np.random.default_rng(14)
    f32 = rng.integers(0, 2**32, 1_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    f32 = f32[~np.isnan(f32)]
    got = oracle.round_from_double("bf16", f32.astype(np.float64))
    want = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, want.view(np.uint16).astype(np.uint32))


# ------------------------------------------------------ single arithmetic ---

def test_f16_sum_and_prod_match_numpy_for_all_a():
    """Every f16 pattern a against a strided sweep of b (16.7M pairs per op)."""
    a = np.repeat(np.arange(65536, dtype=np.uint32), 256)
    b = (np.tile(np.arange(256, dtype=np.uint32), 65536) * 257 + (a % 257)) & 0xFFFF
    fa = a.astype(np.uint16).view(np.float16)
    fb = b.astype(np.uint16).view(np.float16)
    with np.errstate(all="ignore"):
        for op, want in (("sum", fa + fb), ("prod", fa * fb)):
            got = oracle.combine_bits("f16", op, a, b)
            assert _same_bits("f16", got, want.view(np.uint16)).all(), op


def test_f16_sum_matches_exact_rounding_sample():
    """numpy f16 add goes through binary32; cross-check a sample exactly."""
    rng = np.random.default_rng(15)
    a = rng.integers(0, 65536, 3000).astype(np.uint32)
    b = rng.integers(0, 65536, 3000).astype(np.uint32)
    for op in ("sum", "prod"):
        got = oracle.combine_bits("f16", op, a, b)
        for x, y, g in zip(a, b, got):
            w = brute.combine("f16", op, int(x), int(y))
            if w == -1:
                assert _isnan_bits("f16", [g])[0]
            else:
                assert int(g) == w, (op, hex(x), hex(y), hex(int(g)), hex(w))


def test_bf16_sum_and_prod_match_torch():
    rng = np.random.default_rng(16)
    n = 2_000_000
    a = rng.integers(0, 65536, n).astype(np.uint32)
    # b near a in exponent half of the time, so cancellation and ties occur
    b = np.where(rng.random(n) < 0.5, rng.integers(0, 65536, n),
                 (a.astype(np.int64) + rng.integers(-600, 600, n)) & 0xFFFF).astype(np.uint32)
    ta = torch.from_numpy(a.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    for op, want in (("sum", ta + tb), ("prod", ta * tb)):
        got = oracle.combine_bits("bf16", op, a, b)
        w = want.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
        assert _same_bits("bf16", got, w).all(), op


def test_bf16_sum_matches_exact_rounding_sample():
    rng = np.random.default_rng(17)
    a = rng.integers(0, 65536, 3000).astype(np.uint32)
    b = ((a.astype(np.int64) + rng.integers(-300, 300, 3000)) & 0xFFFF).astype(np.uint32)
    for op in ("sum", "prod"):
        got = oracle.combine_bits("bf16", op, a, b)
        for x, y, g in zip(a, b, got):
            w = brute.combine("bf16", op, int(x), int(y))
            if w == -1:
                assert _isnan_bits("bf16", [g])[0]
            else:
                assert int(g) == w, (op, hex(x), hex(y), hex(int(g)), hex(w))


def test_f32_sum_and_prod_match_numpy():
    rng = np.random.default_rng(18)
    n = 2_000_000
    a = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    b = np.where(rng.random(n) < 0.5, rng.integers(0, 2**32, n, dtype=np.uint64),
                 (a.astype(np.int64) + rng.integers(-2**26, 2**26, n)) & 0xFFFFFFFF
                 ).astype(np.uint32)
    fa, fb = a.view(np.float32), b.view(np.float32)
    with np.errstate(all="ignore"):
        for op, want in (("sum", fa + fb), ("prod", fa * fb)):
            got = oracle.combine_bits("f32", op, a, b)
            assert _same_bits("f32", got, want.view(np.uint32)).all(), op


def test_i32_ops_match_numpy():
    rng = np.random.default_rng(19)
    a = rng.integers(-2**31, 2**31, 100000, dtype=np.int64)
    b = rng.integers(-2**31, 2**31, 100000, dtype=np.int64)
    a[:4] = [2**31 - 1, -2**31, -1, 0]
    b[:4] = [1, -1, -2**31, -2**31]
    ua = a.astype(np.int32).view(np.uint32)
    ub = b.astype(np.int32).view(np.uint32)
    wrap = lambda v: ((v + 2**31) % 2**32 - 2**31).astype(np.int32).view(np.uint32)
    assert np.array_equal(oracle.combine_bits("i32", "sum", ua, ub), wrap(a + b))
    assert np.array_equal(oracle.combine_bits("i32", "prod", ua, ub),
                          (a.astype(np.int32) * b.astype(np.int32)).view(np.uint32))
    assert np.array_equal(oracle.combine_bits("i32", "max", ua, ub),
                          np.maximum(a, b).astype(np.int32).view(np.uint32))
    assert np.array_equal(oracle.combine_bits("i32", "min", ua, ub),
                          np.minimum(a, b).astype(np.int32).view(np.uint32))


@pytest.mark.parametrize("dtype", FLOAT_DT)
def test_max_min_zero_nan_inf_rules(dtype):
    """-0 orders below +0 whichever operand comes first; any NaN gives NaN."""
    vals = {"+0": 0.0, "-0": -0.0, "1": 1.0, "-1": -1.0, "inf": np.inf, "-inf": -np.inf}
    enc = {k: int(oracle.round_from_double(dtype, np.array([v]))[0]) for k, v in vals.items()}
    nan = {"f32": 0x7FC00001, "bf16": 0x7FC1, "f16": 0x7E01}[dtype]
    neg_nan = {"f32": 0xFFC00000, "bf16": 0xFFC0, "f16": 0xFE00}[dtype]

    def c(op, x, y):
        return int(oracle.combine_bits(dtype, op, np.array([x]), np.array([y]))[0])

    assert c("max", enc["-0"], enc["+0"]) == enc["+0"]
    assert c("max", enc["+0"], enc["-0"]) == enc["+0"]
    assert c("min", enc["-0"], enc["+0"]) == enc["-0"]
    assert c("min", enc["+0"], enc["-0"]) == enc["-0"]
    assert c("max", enc["-inf"], enc["-1"]) == enc["-1"]
    assert c("min", enc["inf"], enc["1"]) == enc["1"]
    assert c("max", enc["1"], enc["inf"]) == enc["inf"]
    for op in ("max", "min"):
        for other in enc.values():
            for n in (nan, neg_nan):
                assert _isnan_bits(dtype, [c(op, n, other)])[0]
                assert _isnan_bits(dtype, [c(op, other, n)])[0]


# ------------------------------------------------------ whole reductions ---

NS = [1, 2, 3, 5, 8, 16, 17, 64]


@pytest.mark.parametrize("dtype", DT)
def test_closed_form_all_ones(dtype):
    rows, cols, ld, vr, vc = 5, 7, 9, 4, 6
    for n in NS:
        srcs = [_from_values(dtype, np.ones(rows * ld)) for _ in range(n)]
        for op, want in (("sum", n), ("max", 1), ("min", 1), ("prod", 1)):
            for root in sorted({0, n - 1, n // 2}):
                d = _run(srcs, dtype, op, root, rows, cols, ld, vr, vc)
                m = _valid_mask(rows, ld, vr, vc)
                assert np.all(_values(dtype, d)[m] == want), (n, op, root)


@pytest.mark.parametrize("dtype", DT)
def test_closed_form_rank_ids(dtype):
    """S_r = r: Sum = N(N-1)/2, Max = N-1, Min = 0 (every partial sum exact)."""
    rows, cols, ld, vr, vc = 3, 11, 12, 3, 10
    for n in [1, 2, 3, 5, 8, 16, 17, 22]:
        srcs = [_from_values(dtype, np.full(rows * ld, r)) for r in range(n)]
        m = _valid_mask(rows, ld, vr, vc)
        for op, want in (("sum", n * (n - 1) // 2), ("max", n - 1), ("min", 0)):
            for root in sorted({0, n - 1, n // 3}):
                d = _run(srcs, dtype, op, root, rows, cols, ld, vr, vc)
                assert np.all(_values(dtype, d)[m] == want), (n, op, root)


@pytest.mark.parametrize("dtype", DT)
def test_closed_form_prod_powers_of_two(dtype):
    """S_r = 1 + (r mod 2): Prod = 2^(N//2), exact in every type."""
    for n in [2, 3, 8, 16, 17]:
        srcs = [_from_values(dtype, np.full(24, 1 + r % 2)) for r in range(n)]
        for root in (0, n - 1):
            d = _run(srcs, dtype, "prod", root, 4, 6, 6, 4, 6)
            assert np.all(_values(dtype, d) == 2 ** (n // 2))


def _golden_cases():
    path = os.path.join(os.path.dirname(__file__), "golden", "pto_isa_treduce_st_cases.txt")
    cases = []
    for line in open(path):
        line = line.split("#")[0].split()
        if line:
            dt, rows, cols, op, n = line
            cases.append((dt, int(rows), int(cols), op, int(n)))
    return cases


@pytest.mark.parametrize("case", _golden_cases())
def test_pages_system_test_cases(case):
    """Rank r holds base + 100 r; closed-form Sum / Max / Min of the article's tests."""
    dtype, rows, cols, op, n = case
    base = (np.arange(max(rows, 1) * cols) % 4096).astype(np.int64)
    srcs = [_from_values(dtype, base + 100 * r) for r in range(n)]
    want = {"sum": n * base + 50 * n * (n - 1), "max": base + 100 * (n - 1), "min": base}[op]
    for root in (0, n - 1):
        d = _run(srcs, dtype, op, root, rows, cols, cols, rows, cols,
                 dst=_sentinel(dtype, max(rows, 1) * cols))
        if rows == 0:
            assert np.all(_bits(dtype, d) == _bits(dtype, _sentinel(dtype, cols)))
        else:
            assert np.array_equal(_values(dtype, d), want.astype(np.float64))


def test_order_is_root_first_then_ascending():
    """f32 Sum with root 2 of (-1e8, 1, 1e8): (1e8 + -1e8) + 1 = 1.

    Plain rank order (-1e8 + 1) + 1e8 gives 0 instead, because 1 is absorbed
    by 1e8 in binary32; the pages' loop seeds with the root and then skips it.
    """
    srcs = [np.full(4, v, np.float32) for v in (-1e8, 1.0, 1e8)]
    d = _run(srcs, "f32", "sum", 2, 1, 4, 4, 1, 4)
    assert np.all(d == 1.0)
    d0 = _run(srcs, "f32", "sum", 0, 1, 4, 4, 1, 4)
    assert np.all(d0 == 0.0)


def _random_bits(dtype, rng, n):
    if dtype == "i32":
        v = rng.integers(-2**31, 2**31, n, dtype=np.int64)
        small = rng.integers(-50, 50, n)
        return np.where(rng.random(n) < 0.5, small, v).astype(np.int32)
    if dtype == "f32":
        v = (rng.standard_normal(n) * np.exp2(rng.integers(-10, 10, n))).astype(np.float32)
        raw = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        v = np.where(rng.random(n) < 0.1, raw, v).astype(np.float32)
        v[rng.random(n) < 0.05] = 0.0
        v[rng.random(n) < 0.05] = -0.0
        return v
    raw = rng.integers(0, 65536, n).astype(np.uint16)
    v = rng.standard_normal(n).astype(np.float32)
    if dtype == "f16":
        soft = v.astype(np.float16).view(np.uint16)
    else:
        soft = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = np.where(rng.random(n) < 0.2, raw, soft).astype(np.uint16)
    out[rng.random(n) < 0.05] = 0x0000
    out[rng.random(n) < 0.05] = 0x8000
    return out


def _to_brute(dtype, buf):
    if dtype == "i32":
        return [int(x) for x in buf]
    return [int(x) for x in _bits(dtype, buf)]


@pytest.mark.parametrize("dtype", DT)
def test_brute_force_tiny(dtype):
    rng = np.random.default_rng({"f32": 1, "bf16": 2, "f16": 3, "i32": 4}[dtype])
    for case in range(24):
        n = int(rng.choice([1, 2, 3, 4, 5, 8, 17]))
        rows = int(rng.integers(1, 5))
        cols = int(rng.integers(1, 7))
        ld = cols + int(rng.integers(0, 3))
        vr = int(rng.integers(0, rows + 1))
        vc = int(rng.integers(0, cols + 1))
        root = int(rng.integers(0, n))
        op = ["sum", "max", "min", "prod"][case % 4]
        size = (rows - 1) * ld + cols
        srcs = [_random_bits(dtype, rng, size) for _ in range(n)]
        d = _sentinel(dtype, size)
        oracle.treduce(srcs, d, root=root, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                       valid_rows=vr, valid_cols=vc)
        want = brute.treduce([_to_brute(dtype, s) for s in srcs], root, dtype, op, ld, vr, vc)
        got = _bits(dtype, d)
        sent = _bits(dtype, _sentinel(dtype, size))
        for k in range(size):
            i, j = divmod(k, ld)
            if (i, j) in want:
                w = want[(i, j)]
                if dtype == "i32":
                    assert int(d[k]) == w, (case, n, op, root, i, j)
                elif w == -1:
                    assert _isnan_bits(dtype, [got[k]])[0], (case, op, i, j)
                elif n == 1:
                    assert int(got[k]) == w
                else:
                    assert int(got[k]) == w, (case, n, op, root, i, j, hex(int(got[k])), hex(w))
            else:
                assert got[k] == sent[k], (case, i, j)


@pytest.mark.parametrize("dtype", DT)
def test_banded_oracle_matches_brute_force(dtype):
    """The row-band driver used on full-size workloads covers every valid row
    exactly once: checked against the brute force on a ragged rectangle whose
    rows do not divide evenly into the bands (including bands of one row)."""
    rng = np.random.default_rng({"f32": 11, "bf16": 12, "f16": 13, "i32": 14}[dtype])
    for rows, cols, ld, vr, vc, threads in ((37, 23, 29, 35, 21, 8), (9, 5, 5, 9, 5, 4),
                                            (20, 7, 9, 19, 6, 3)):
        n, root = 5, 2
        size = (rows - 1) * ld + cols
        srcs = [_random_bits(dtype, rng, size) for _ in range(n)]
        d = _sentinel(dtype, size)
        oracle.treduce_banded(srcs, d, root=root, dtype=dtype, op="sum", rows=rows, cols=cols,
                              ld=ld, valid_rows=vr, valid_cols=vc, threads=threads)
        want = brute.treduce([_to_brute(dtype, s) for s in srcs], root, dtype, "sum", ld, vr,
                             vc)
        got = _bits(dtype, d)
        sent = _bits(dtype, _sentinel(dtype, 1))[0]
        for k in range(size):
            i, j = divmod(k, ld)
            if (i, j) not in want:
                assert got[k] == sent, (rows, i, j)
            elif dtype == "i32":
                assert int(d[k]) == want[(i, j)], (rows, i, j)
            elif want[(i, j)] == -1:
                assert _isnan_bits(dtype, [got[k]])[0], (rows, i, j)
            else:
                assert int(got[k]) == want[(i, j)], (rows, i, j)


def test_single_rank_is_a_bitwise_copy():
    """N == 1: the root's bits are stored unchanged, NaN payloads included."""
    for dtype in DT:
        rng = np.random.default_rng(5)
        if dtype in ("f32", "i32"):
            s = rng.integers(0, 2**32, 300, dtype=np.uint64).astype(np.uint32)
            s[:3] = [0x7F800001, 0xFFC01234, 0x80000000]
            s = s.view(STORAGE[dtype])
        else:
            s = rng.integers(0, 65536, 300).astype(np.uint16)
            s[:3] = [0x7C01, 0xFE55, 0x7F81]
        for op in ("sum", "max", "min", "prod"):
            d = _run([s], dtype, op, 0, 10, 30, 30, 10, 30)
            assert np.array_equal(_bits(dtype, d), _bits(dtype, s))


def test_empty_region_writes_nothing():
    s = [np.ones(64, np.float32)] * 3
    for vr, vc, rows in ((0, 8, 8), (8, 0, 8), (0, 0, 0)):
        d = _sentinel("f32", 64)
        oracle.treduce(s, d, root=1, dtype="f32", op="sum", rows=rows, cols=8, ld=8,
                       valid_rows=vr, valid_cols=vc)
        assert np.all(d.view(np.int32) == -1)


@pytest.mark.parametrize("dtype", DT)
def test_outside_valid_untouched_and_never_read(dtype):
    """Sentinel dst and guard bands stay intact; poisoned source cells outside
    the valid rectangle never reach an output."""
    rng = np.random.default_rng(6)
    rows, cols, ld, vr, vc, n = 9, 13, 16, 7, 10, 5
    guard = 37
    size = rows * ld
    clean = [_random_bits(dtype, rng, size) for _ in range(n)]
    poison = {"f32": np.float32(np.nan), "i32": np.int32(-2**31), "bf16": np.uint16(0x7FC1),
              "f16": np.uint16(0x7E01)}[dtype]
    m = _valid_mask(rows, ld, vr, vc)
    dirty = [np.where(m, s, poison).astype(s.dtype) for s in clean]
    for op in ("sum", "max", "min"):
        big = _sentinel(dtype, size + 2 * guard)
        view = big[guard:guard + size]
        oracle.treduce(dirty, view, root=2, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                       valid_rows=vr, valid_cols=vc)
        ref = _run(clean, dtype, op, 2, rows, cols, ld, vr, vc)
        sent = _bits(dtype, _sentinel(dtype, size + 2 * guard))
        got = _bits(dtype, big)
        assert np.array_equal(got[:guard], sent[:guard])
        assert np.array_equal(got[guard + size:], sent[guard + size:])
        assert np.array_equal(got[guard:guard + size][~m], sent[guard:guard + size][~m])
        assert _same_bits(dtype, _bits(dtype, view)[m], _bits(dtype, ref)[m]).all()


@pytest.mark.parametrize("dtype,op", [("i32", "sum"), ("i32", "max"), ("i32", "min"),
                                      ("i32", "prod"), ("f32", "max"), ("f32", "min"),
                                      ("bf16", "max"), ("f16", "min")])
def test_order_free_ops_ignore_permutation_and_root(dtype, op):
    rng = np.random.default_rng(7)
    n, size = 9, 500
    srcs = [_random_bits(dtype, rng, size) for _ in range(n)]
    ref = _run(srcs, dtype, op, 0, 1, size, size, 1, size)
    for trial in range(4):
        perm = rng.permutation(n)
        d = _run([srcs[p] for p in perm], dtype, op, int(rng.integers(0, n)), 1, size, size, 1,
                 size)
        assert _same_bits(dtype, _bits(dtype, d), _bits(dtype, ref)).all()
    if dtype == "i32":
        stack = np.stack([s.astype(np.int64) for s in srcs])
        lib = {"sum": lambda: ((stack.sum(0) + 2**31) % 2**32 - 2**31),
               "max": lambda: stack.max(0), "min": lambda: stack.min(0),
               "prod": None}[op]
        if lib is not None:
            assert np.array_equal(ref.astype(np.int64), lib())


def test_float_max_min_match_numpy_without_ties():
    rng = np.random.default_rng(8)
    srcs = [rng.standard_normal(4000).astype(np.float32) for _ in range(6)]
    stack = np.stack(srcs)
    for op, fn in (("max", np.max), ("min", np.min)):
        d = _run(srcs, "f32", op, 3, 40, 100, 100, 40, 100)
        assert np.array_equal(d, fn(stack, axis=0))


def test_allreduce_inplace_writes_every_buffer():
    rng = np.random.default_rng(9)
    rows, cols, ld, vr, vc, n = 6, 10, 12, 5, 9, 4
    bufs = [rng.standard_normal(rows * ld).astype(np.float32) for _ in range(n)]
    before = [b.copy() for b in bufs]
    want = _run(before, "f32", "sum", 0, rows, cols, ld, vr, vc)
    oracle.allreduce_inplace(bufs, root=0, dtype="f32", op="sum", rows=rows, cols=cols, ld=ld,
                             valid_rows=vr, valid_cols=vc)
    m = _valid_mask(rows, ld, vr, vc)
    for b, b0 in zip(bufs, before):
        assert np.array_equal(b[m], want[m])
        assert np.array_equal(b[~m], b0[~m])


def test_rejects_invalid_arguments():
    s = [np.zeros(16, np.float32)] * 2
    d = np.zeros(16, np.float32)
    bad = [dict(root=2), dict(root=-1), dict(valid_rows=5), dict(valid_cols=5), dict(cols=5),
           dict(rows=-1, valid_rows=-1)]
    for kw in bad:
        args = dict(root=0, dtype="f32", op="sum", rows=4, cols=4, ld=4, valid_rows=4,
                    valid_cols=4)
        args.update(kw)
        with pytest.raises(ValueError):
            oracle.treduce(s, d, **args)
