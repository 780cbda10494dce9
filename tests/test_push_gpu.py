"""GPU parity of push-with-add ("Distributed Operators (N6)", pld.tensor.put /
remote_store with atomic = kAdd) through the C ABI.

* Default (fold, then push): each element's N sources are folded in rank
  order as the reduction folds them with root 0, and the fold is added into
  dst by one atomic.  With no concurrent push the result has one possible
  value: dst + fold rounded once to the element type.  Compared bit for bit
  with the oracle (its fold, then its one combine step).
* PTORED_ACC_PER_RANK: N atomics per element in a varying order.  With
  inputs whose every partial sum is exact (small integers, or small
  multiples of the smallest subnormal) every order gives the same bits, so
  this path too is compared bit for bit with the oracle's rank-order sums;
  this covers the 16-bit pairing across lanes and slices, the half-word
  compare-and-swap, heads, row remainders and odd pitches exactly.
* Subnormal sums: both paths keep them (no flush) -- checked exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W
from tests.gpu_helpers import DevBuf, ESIZE, bits, compare, say, sentinel, valid_mask
from tests.test_collectives_gpu import _finite_values

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16", "i32"]


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


def _u32(dtype, a):
    return bits(dtype, a).astype(np.uint32)


def _fold_then_add(srcs, d0, dtype, rows, cols, ld, vr, vc):
    """The oracle's value of the default push: dst + fold(srcs), the fold in
    rank order (root 0) and the final addition rounded once."""
    size = d0.size
    fold = sentinel(dtype, size)
    oracle.treduce([s.copy() for s in srcs], fold, root=0, dtype=dtype, op="sum", rows=rows,
                   cols=cols, ld=ld, valid_rows=vr, valid_cols=vc)
    m = valid_mask(rows, ld, vr, vc, size)
    want = d0.copy()
    summed = oracle.combine_bits(dtype, "sum", _u32(dtype, d0[m]), _u32(dtype, fold[m]))
    want[m] = summed.astype(np.uint16 if ESIZE[dtype] == 2 else np.uint32).view(want.dtype)
    return want, m


def _run_push(srcs, d0, dtype, rows, cols, ld, vr, vc, offs, doff, flags, label):
    sb = _upload(srcs, offs)
    db = _upload([d0], [doff])[0]
    say(label, f"dtype={dtype} N={len(srcs)} {rows}x{cols} ld={ld} valid={vr}x{vc} "
               f"offs={offs[:3]} doff={doff} flags={flags:#x}")
    st = B.ptored_accumulate_add([b.ptr for b in sb], len(srcs), db.ptr, rows, cols, ld, vr, vc,
                                 B.DTYPES[dtype], B.tuning(flags=flags), _stream())
    torch.cuda.synchronize()
    assert st == 0, B.ptored_status_string(st)
    assert db.guards_intact(), label
    return db.download(dtype)


SHAPE_FLAGS = [0, B.PTORED_FORCE_ELEMENTWISE, B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES,
               B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, B.PTORED_FORCE_RUNTIME_N]


def _case_shape(rng, case, es):
    n = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 33]))
    rows = int(rng.integers(1, 24))
    cols = int(rng.integers(1, 900))
    ld = cols + int(rng.choice([0, 1, 3, 8, 64]))  # 1 and 3: odd pitches
    vr, vc = int(rng.integers(1, rows + 1)), int(rng.integers(1, cols + 1))
    kind = case % 4
    if kind == 0:  # every buffer at one offset inside a 16-byte block: heads
        lead = int(rng.integers(0, 16 // es)) * es
        offs, doff = [lead] * n, lead
    elif kind == 1:  # sources anywhere, dst at 2 mod 4 (16-bit) or 4 mod 16
        offs = [int(rng.integers(0, 64 // es)) * es for _ in range(n)]
        doff = 2 if es == 2 else 4
    else:
        offs, doff = [0] * n, 0
    flags = SHAPE_FLAGS[case % len(SHAPE_FLAGS)]
    return n, rows, cols, ld, vr, vc, offs, doff, flags


@pytest.mark.parametrize("dtype", DT)
def test_push_fold_is_bit_exact(dtype):
    """Default push-with-add equals dst + fold(srcs), bit for bit, over random
    shapes, offsets, pitches and every forced kernel family and walk."""
    rng = np.random.default_rng({"f32": 91, "bf16": 92, "f16": 93, "i32": 94}[dtype])
    es = ESIZE[dtype]
    for case in range(30):
        n, rows, cols, ld, vr, vc, offs, doff, flags = _case_shape(rng, case, es)
        size = (rows - 1) * ld + cols
        srcs = [_finite_values(dtype, rng, size) for _ in range(n)]
        d0 = _finite_values(dtype, rng, size)
        got = _run_push(srcs, d0, dtype, rows, cols, ld, vr, vc, offs, doff, flags,
                        f"push fold#{case}")
        want, m = _fold_then_add(srcs, d0, dtype, rows, cols, ld, vr, vc)
        assert np.array_equal(got[~m].view(np.uint8), d0[~m].view(np.uint8)), case
        ok = compare(dtype, got, want)
        assert ok.all(), (case, int((~ok).sum()), int(np.argmin(ok)))


def _small_integers(dtype, rng, n):
    """Values whose sums of up to 34 terms are exact in the element type."""
    if dtype == "i32":
        return rng.integers(-2**20, 2**20, n).astype(np.int32)
    if dtype == "f32":
        return rng.integers(-2**12, 2**12, n).astype(np.float32)
    if dtype == "f16":
        return rng.integers(-32, 33, n).astype(np.float16).view(np.uint16)
    v = rng.integers(-4, 5, n).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rank_order_sum(srcs, d0, dtype, rows, cols, ld, vr, vc):
    want = d0.copy()
    oracle.accumulate_add([s.copy() for s in srcs], want, dtype=dtype, rows=rows, cols=cols,
                          ld=ld, valid_rows=vr, valid_cols=vc)
    return want


@pytest.mark.parametrize("mode", ["per_rank", "fold"])
@pytest.mark.parametrize("dtype", DT)
def test_push_exact_sums_bit_for_bit(dtype, mode):
    """Inputs whose every partial sum is exact: both paths, in any order of
    the additions, give the oracle's rank-order sum bit for bit.  Shapes
    include odd pitches, dst at 2 mod 4, heads and row remainders on the
    vector path and the element-wise path (with its pairing of 16-bit
    neighbours across lanes and 64-element slices)."""
    rng = np.random.default_rng({"f32": 95, "bf16": 96, "f16": 97, "i32": 98}[dtype]
                                + (0 if mode == "fold" else 10))
    es = ESIZE[dtype]
    extra = B.PTORED_ACC_PER_RANK if mode == "per_rank" else 0
    for case in range(30):
        n, rows, cols, ld, vr, vc, offs, doff, flags = _case_shape(rng, case, es)
        size = (rows - 1) * ld + cols
        srcs = [_small_integers(dtype, rng, size) for _ in range(n)]
        d0 = _small_integers(dtype, rng, size)
        got = _run_push(srcs, d0, dtype, rows, cols, ld, vr, vc, offs, doff, flags | extra,
                        f"push exact {mode}#{case}")
        want = _rank_order_sum(srcs, d0, dtype, rows, cols, ld, vr, vc)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), case


MIN_SUB = {"f32": 2.0 ** -149, "f16": 2.0 ** -24, "bf16": 2.0 ** -133}


def _subnormals(dtype, rng, n):
    """Small integer multiples of the smallest subnormal (|k| <= 8): every sum
    of up to 10 of them is an exact subnormal (or zero)."""
    k = rng.integers(-8, 9, n).astype(np.float64)
    bits_ = oracle.round_from_double(dtype, k * MIN_SUB[dtype])
    return bits_.astype(np.uint32).view(np.float32) if dtype == "f32" else \
        bits_.astype(np.uint16)


@pytest.mark.parametrize("mode", ["per_rank", "fold"])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_push_keeps_subnormal_sums(dtype, mode):
    """Sums that stay in the subnormal range are kept, not flushed to zero:
    sources and dst are small multiples of the smallest subnormal, so every
    order of the additions gives the same exact sum."""
    rng = np.random.default_rng({"f32": 101, "bf16": 102, "f16": 103}[dtype])
    extra = B.PTORED_ACC_PER_RANK if mode == "per_rank" else 0
    for case, (n, rows, cols, ld, flags) in enumerate([
            (8, 64, 1024, 1024, 0), (3, 7, 301, 304, 0), (5, 9, 77, 77, B.PTORED_FORCE_ELEMENTWISE),
            (9, 5, 200, 203, 0)]):
        size = (rows - 1) * ld + cols
        srcs = [_subnormals(dtype, rng, size) for _ in range(n)]
        d0 = _subnormals(dtype, rng, size)
        got = _run_push(srcs, d0, dtype, rows, cols, ld, rows, cols, [0] * n, 0, flags | extra,
                        f"push subnormal {mode}#{case}")
        want = _rank_order_sum(srcs, d0, dtype, rows, cols, ld, rows, cols)
        m = valid_mask(rows, ld, rows, cols, size)
        nonzero = oracle.to_double(dtype, _u32(dtype, want[m])) != 0.0
        assert nonzero.mean() > 0.5  # the case really has subnormal sums
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), case


@pytest.mark.parametrize("name", ["n8_bf16_8192x8192", "n8_f16_8192x12288_valid8191x12287"])
def test_push_fold_full_size(name):
    """Default push-with-add over a full-size 16-bit workload (sources from
    the workload, dst one more rank's draw; the saturated f16 entries make
    some sums overflow to +-Inf or NaN, compared by NaN-ness): every valid
    element equals dst + fold(srcs), everything else unchanged."""
    w = W.WORKLOADS[name]
    srcs = W.make_sources(w)
    d0 = W.draw(w.recipe, w.buffer_elems, w.seed_base + 100)
    got = _run_push(srcs, d0, w.dtype, w.rows, w.cols, w.ld, w.valid_rows, w.valid_cols,
                    [0] * w.nranks, 0, 0, f"push full {name}")
    want, m = _fold_then_add(srcs, d0, w.dtype, w.rows, w.cols, w.ld, w.valid_rows,
                             w.valid_cols)
    assert np.array_equal(got[~m].view(np.uint8), d0[~m].view(np.uint8))
    ok = compare(w.dtype, got[m], want[m])
    assert ok.all(), (int((~ok).sum()), int(np.argmin(ok)))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_push_fold_special_values(dtype):
    """The default push with arbitrary bit patterns in the sources and in dst
    (NaN, +-Inf, subnormals, signed zeros among them): dst + fold(srcs)
    bit for bit, NaN by NaN-ness -- the atomic unit's special cases (-0 plus
    -0, Inf minus Inf, subnormal sums) match IEEE addition rounded once."""
    from tests.test_parity_gpu import _rand_elems

    rng = np.random.default_rng({"f32": 111, "bf16": 112, "f16": 113}[dtype])
    for case, (n, rows, cols, ld, flags) in enumerate([
            (5, 33, 700, 704, 0), (3, 17, 501, 503, 0), (8, 9, 300, 300, B.PTORED_FORCE_ELEMENTWISE),
            (2, 64, 1024, 1024, 0)]):
        size = (rows - 1) * ld + cols
        srcs = [_rand_elems(dtype, rng, size, wild=0.3) for _ in range(n)]
        d0 = _rand_elems(dtype, rng, size, wild=0.3)
        # -0 in dst against folds of -0 (every source -0 there): -0 + -0 must stay -0
        z = rng.random(size) < 0.02
        neg0 = np.float32(-0.0) if dtype == "f32" else np.uint16(0x8000)
        for s_ in srcs + [d0]:
            s_[z] = neg0
        got = _run_push(srcs, d0, dtype, rows, cols, ld, rows, cols, [0] * n, 0, flags,
                        f"push special#{case}")
        want, m = _fold_then_add(srcs, d0, dtype, rows, cols, ld, rows, cols)
        ok = compare(dtype, got, want)
        assert ok.all(), (case, int((~ok).sum()), int(np.argmin(ok)))
