"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: bit-exact for every dtype and op (i32; Max/Min; float Sum/Prod in the
fold order root-first-then-ascending, which the kernels keep), NaN compared
by NaN-ness.  Cells outside the valid rectangle and the guard bands around
dst keep their sentinel bytes; sources are never written.
"""

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W
from tests.gpu_helpers import (compare, oracle_reduce, oracle_reduce_banded, run_gpu, say,
                               sentinel, valid_mask, DevBuf, ESIZE, STORAGE)

pytestmark = pytest.mark.gpu

DT = ["f32", "bf16", "f16", "i32"]
OPS = ["sum", "max", "min", "prod"]


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _rand_elems(dtype, rng, n, wild=0.15):
    """Values of the kind the reduction meets, with a share of arbitrary bit
    patterns (NaN, Inf, subnormals, signed zeros) mixed in."""
    if dtype == "i32":
        v = rng.integers(-2**31, 2**31, n, dtype=np.int64)
        small = rng.integers(-1000, 1000, n)
        return np.where(rng.random(n) < 0.5, small, v).astype(np.int32)
    g = rng.standard_normal(n).astype(np.float32) * np.exp2(rng.integers(-8, 8, n)).astype(
        np.float32)
    if dtype == "f32":
        raw = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        out = np.where(rng.random(n) < wild, raw, g).astype(np.float32)
        out[rng.random(n) < 0.02] = 0.0
        out[rng.random(n) < 0.02] = -0.0
        return out
    if dtype == "f16":
        soft = g.astype(np.float16).view(np.uint16)
    else:
        soft = torch.from_numpy(g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raw = rng.integers(0, 65536, n).astype(np.uint16)
    out = np.where(rng.random(n) < wild, raw, soft).astype(np.uint16)
    out[rng.random(n) < 0.02] = 0x0000
    out[rng.random(n) < 0.02] = 0x8000
    return out


def _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, alias=-1, label=""):
    size = (rows - 1) * ld + cols if rows > 0 else 0
    got = dst.download(dtype)
    want = oracle_reduce(srcs, dtype, op, root, rows, cols, ld, vr, vc,
                         lambda n: sentinel(dtype, n) if alias < 0 else srcs[alias][:n].copy())
    m = valid_mask(rows, ld, vr, vc, max(size, 1)) if size else np.zeros(1, bool)
    ok = compare(dtype, got, want)
    bad = np.flatnonzero(~ok & m)
    assert bad.size == 0, (label, bad[:8], got[bad[:4]], want[bad[:4]])
    # outside the valid rectangle: untouched bytes
    outside = ~m
    if alias < 0:
        assert np.array_equal(got.view(np.uint8).reshape(-1, ESIZE[dtype])[outside],
                              np.full((outside.sum(), ESIZE[dtype]), 0xFF, np.uint8)), label
    else:
        assert np.array_equal(got[outside].view(np.uint8),
                              srcs[alias][:max(size, 1)][outside].view(np.uint8)), label
    assert dst.guards_intact(), label
    for r, b in enumerate(bufs):
        if r != alias:
            assert np.array_equal(b.download(dtype).view(np.uint8),
                                  srcs[r][:max(size, 1)].view(np.uint8)), (label, "src", r)


VARIANTS = [
    ("auto", 0, 0),
    ("elementwise", B.PTORED_FORCE_ELEMENTWISE, 0),
    ("rows", B.PTORED_FORCE_ROWS, 0),
    ("flat", B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, 0),
    ("row_tiles", B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, 0),
    ("full_occupancy", B.PTORED_FULL_OCCUPANCY, 0),
    ("runtime_n", B.PTORED_FORCE_RUNTIME_N, 0),
    ("lds_pingpong", B.PTORED_LDS_PINGPONG, 0),
    ("persistent_noremap", B.PTORED_NO_XCD_REMAP, 2),
    ("one_block_per_cu", 0, 1),
    ("persistent_occupancy", 0, -1),
]


@pytest.mark.parametrize("dtype", DT)
def test_random_small_cases(dtype):
    """Tiny shapes, every op, N from 1 to 64, any root, odd pitches, misaligned
    pointers, sub-rectangles and every kernel variant."""
    rng = np.random.default_rng({"f32": 11, "bf16": 12, "f16": 13, "i32": 14}[dtype])
    es = ESIZE[dtype]
    for case in range(40):
        n = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 33, 64]))
        rows = int(rng.integers(1, 9))
        cols = int(rng.integers(1, 80))
        ld = cols + int(rng.choice([0, 0, 1, 3, 8, 16]))
        vr = int(rng.integers(1, rows + 1))
        vc = int(rng.integers(1, cols + 1))
        root = int(rng.choice([0, n - 1, int(rng.integers(0, n))]))
        op = OPS[case % 4]
        vname, flags, bpc = VARIANTS[case % len(VARIANTS)]
        aligned = rng.random() < 0.6
        offs = [0 if aligned else int(rng.integers(0, 8)) * es for _ in range(n)]
        dst_off = 0 if aligned else int(rng.integers(0, 8)) * es
        size = (rows - 1) * ld + cols
        srcs = [_rand_elems(dtype, rng, size) for _ in range(n)]
        t = B.tuning(flags=flags, blocks_per_cu=bpc)
        label = f"small#{case} {vname}"
        dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc, offsets=offs,
                                dst_offset=dst_off, tuning=t, label=label)
        assert st == 0, B.ptored_status_string(st)
        _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, label=label)


# Shapes for buffers that all start `lead` bytes past a 16-byte boundary
# (2-D pitches are multiples of 16 bytes for every element size; the spans'
# pitches are not, which matters when the row walk is forced).
LEAD_SHAPES = [
    # rows, cols, ld, valid_rows, valid_cols
    (1, 5003, 5003, 1, 5003),      # one contiguous span
    (40, 256, 256, 40, 256),       # rows back to back: contiguous
    (33, 1030, 1040, 31, 1029),    # 2-D, ragged row ends
    (9, 4100, 4104, 9, 4099),      # row tiles: 4+ chunks per row
    (5, 9, 16, 5, 8),              # rows of one head, at most one slot and a tail
    (1, 7, 7, 1, 7),               # tiny: vector only when lead + 7 elements reach 16 bytes
    (1, 1, 1, 1, 1),               # one element: never reaches the boundary (element-wise)
]


@pytest.mark.parametrize("dtype", DT)
def test_common_lead_keeps_vector_path(dtype):
    """Every buffer the same number of bytes past a 16-byte boundary: the
    vector kernels with a head per row, against the oracle, in every walk,
    with windows, the runtime rank loop, the LDS variant and in place."""
    rng = np.random.default_rng({"f32": 71, "bf16": 72, "f16": 73, "i32": 74}[dtype])
    es = ESIZE[dtype]
    leads = list(range(es, 16, es))
    variants = [("auto", 0, 0), ("flat", B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, 0),
                ("row_tiles", B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, 0),
                ("runtime_n", B.PTORED_FORCE_RUNTIME_N, 0), ("lds", B.PTORED_LDS_PINGPONG, 0),
                ("windows", 0, 1008), ("windows_rows", B.PTORED_FORCE_ROWS, 4096 + 48)]
    case = 0
    for rows, cols, ld, vr, vc in LEAD_SHAPES:
        for vi, (vname, flags, mlb) in enumerate(variants):
            lead = leads[(case * 3 + vi) % len(leads)]
            n = int(rng.choice([1, 2, 3, 8, 16, 20]))
            root = int(rng.integers(0, n))
            op = OPS[case % 4]
            offs = [lead + 16 * int(rng.integers(0, 4)) for _ in range(n)]
            dst_off = lead + 16 * int(rng.integers(0, 4))
            alias = int(rng.integers(0, n)) if case % 5 == 4 else -1
            size = (rows - 1) * ld + cols
            srcs = [_rand_elems(dtype, rng, size) for _ in range(n)]
            t = B.tuning(flags=flags, max_launch_bytes=mlb)
            label = f"lead#{case} lead={lead} {vname} {rows}x{cols} ld={ld} valid={vr}x{vc}"
            st_plan, info = B.ptored_treduce_plan(
                [0x1000000 + o for o in offs], n, root,
                0x9000000 + (offs[alias] if alias >= 0 else dst_off), rows, cols, ld, vr, vc,
                B.DTYPES[dtype], B.OPS[op], t)
            assert st_plan == 0
            contig = (vc == ld or vr == 1) and not flags & B.PTORED_FORCE_ROWS
            row_bytes = ((vc if vr == 1 else vr * ld) if contig else vc) * es
            # else the element-wise kernel: a row that never reaches the
            # boundary; rows whose pitch is off the 16-byte grid number their
            # slots from each row's start (element-wise only through the LDS
            # variant, which keeps the shared-offset rule)
            if contig or (ld * es) % 16 == 0:
                vector = lead + row_bytes >= 16
            else:
                vector = not (flags & B.PTORED_LDS_PINGPONG and n > 1)
            assert (B.PATHS[info.path] != "elementwise") == vector, label
            dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc, offsets=offs,
                                    dst_offset=dst_off, tuning=t, alias=alias, label=label)
            assert st == 0, B.ptored_status_string(st)
            _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, alias=alias,
                   label=label)
            case += 1


@pytest.mark.parametrize("dtype", DT)
def test_common_line_offset(dtype):
    """Every buffer at the same byte offset (views at one element offset into
    larger allocations): slots numbered from the coarsest of a 1 KiB, 128-byte
    or 16-byte boundary that the pitch keeps, the ones before the data
    skipped, a head when the offset is inside a 16-byte block.  Every walk,
    windows, the LDS variant, in place."""
    rng = np.random.default_rng({"f32": 171, "bf16": 172, "f16": 173, "i32": 174}[dtype])
    es = ESIZE[dtype]
    offsets = [o for o in (es, 16, 16 + es, 36, 64, 100, 124, 126, 132, 520, 1020, 1022)
               if o % es == 0]
    shapes = LEAD_SHAPES[:5] + [(33, 1000, 1024, 31, 999), (7, 3000, 3072, 7, 2999)]
    variants = [("auto", 0, 0), ("flat", B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, 0),
                ("row_tiles", B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, 0),
                ("lds", B.PTORED_LDS_PINGPONG, 0), ("windows", 0, 1008),
                ("windows_16", 0, 16)]
    case = 0
    for rows, cols, ld, vr, vc in shapes:
        for vi, (vname, flags, mlb) in enumerate(variants):
            off = offsets[(case * 5 + vi) % len(offsets)]
            n = int(rng.choice([1, 2, 5, 8, 16]))
            root = int(rng.integers(0, n))
            op = OPS[case % 4]
            alias = int(rng.integers(0, n)) if case % 7 == 6 else -1
            size = (rows - 1) * ld + cols
            if mlb == 16 and size * es > 1 << 16:
                continue  # 16-byte windows: small buffers only
            srcs = [_rand_elems(dtype, rng, size) for _ in range(n)]
            t = B.tuning(flags=flags, max_launch_bytes=mlb)
            label = f"line#{case} off={off} {vname} {rows}x{cols} ld={ld} valid={vr}x{vc} N={n}"
            st_plan, info = B.ptored_treduce_plan(
                [0x1000000 + off] * n, n, root, 0x9000000 + off, rows, cols, ld, vr, vc,
                B.DTYPES[dtype], B.OPS[op], t)
            assert st_plan == 0
            contig = (vc == ld or vr == 1) and not flags & B.PTORED_FORCE_ROWS
            if B.PATHS[info.path] != "elementwise":
                if contig or (ld * es) % 16 == 0:
                    origin = next(a for a in (1024, 128, 16) if contig or (ld * es) % a == 0)
                    assert info.lead == off % origin, label
                else:
                    assert info.lead == 0, label  # slots from each row's start
            dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc,
                                    offsets=[off] * n, dst_offset=off, tuning=t, alias=alias,
                                    label=label)
            assert st == 0, B.ptored_status_string(st)
            _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, alias=alias,
                   label=label)
            case += 1


# Rows whose last few whole slots spill into the tail tiles (fewer than half a
# row tile past the last whole one), with and without a lead: (rows, cols,
# ld, valid_rows, valid_cols, byte offset of every buffer).
SPILL_SHAPES = [
    (37, 1040, 1048, 37, 1040, 0),    # f32: 260 slots = 4 tiles + 4; 16-bit: 2 + 2
    (9, 1040, 1088, 9, 1036, 0),      # remainder bytes after the spill slots
    (4000, 272, 288, 4000, 260, 64),  # one whole tile and a short spill, many rows
    (61, 12288, 12288, 61, 12287, 64),  # the ragged f16 shape at a 64-byte offset
    (5, 300, 320, 5, 260, 36),        # a head, whole tiles, spill and a remainder
]


# Shapes for the unaligned vector path: buffers at different offsets within
# 16 bytes, and row pitches off the 16-byte grid (the last two).
UNALIGNED_SHAPES = [
    # rows, cols, ld, valid_rows, valid_cols
    (1, 70001, 70001, 1, 70001),   # one contiguous span
    (41, 1040, 1040, 41, 1040),    # rows back to back: contiguous
    (37, 1024, 1040, 35, 1021),    # 2-D, pitch on the 16-byte grid, ragged row ends
    (9, 4100, 4112, 9, 4099),      # row tiles: 4+ chunks per row
    (37, 1030, 1031, 35, 1029),    # odd pitch: each row at its own offset
    (12, 4099, 4101, 12, 4099),    # odd pitch, full rows
]


@pytest.mark.parametrize("dtype", DT)
def test_unaligned_vector_path(dtype):
    """Buffers at different offsets within 16 bytes take the vector kernels
    with dst's alignment (the other buffers read unaligned), and odd row
    pitches number each row's slots from its start; against the oracle in
    every walk, with windows, the runtime rank loop and in place.  The plan
    is checked to be the vector path, except through the LDS variant."""
    rng = np.random.default_rng({"f32": 181, "bf16": 182, "f16": 183, "i32": 184}[dtype])
    es = ESIZE[dtype]
    variants = [("auto", 0, 0), ("flat", B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, 0),
                ("row_tiles", B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, 0),
                ("runtime_n", B.PTORED_FORCE_RUNTIME_N, 0), ("windows", 0, 1008),
                ("windows_rows", B.PTORED_FORCE_ROWS, 4096 + 48), ("lds", B.PTORED_LDS_PINGPONG, 0)]
    case = 0
    for rows, cols, ld, vr, vc in UNALIGNED_SHAPES:
        for vname, flags, mlb in variants:
            n = int(rng.choice([1, 2, 3, 8, 16, 20]))
            root = int(rng.integers(0, n))
            op = OPS[case % 4]
            offs = [es * int(rng.integers(0, 16 // es)) + 16 * int(rng.integers(0, 4))
                    for _ in range(n)]
            if len({o % 16 for o in offs}) == 1 and n > 1:
                offs[-1] = (offs[-1] + es) % 64  # at least two offsets within 16 bytes
            dst_off = es * int(rng.integers(0, 1024 // es))
            alias = int(rng.integers(0, n)) if case % 6 == 5 else -1
            size = (rows - 1) * ld + cols
            srcs = [_rand_elems(dtype, rng, size) for _ in range(n)]
            t = B.tuning(flags=flags, max_launch_bytes=mlb)
            label = (f"unaligned#{case} {vname} {rows}x{cols} ld={ld} valid={vr}x{vc} N={n} "
                     f"offs={offs[:4]} dst={dst_off if alias < 0 else offs[alias]}")
            d_off = offs[alias] if alias >= 0 else dst_off
            st_plan, info = B.ptored_treduce_plan(
                [0x1000000 + o for o in offs], n, root, 0x9000000 + d_off, rows, cols, ld, vr,
                vc, B.DTYPES[dtype], B.OPS[op], t)
            assert st_plan == 0
            contig = (vc == ld or vr == 1) and not flags & B.PTORED_FORCE_ROWS
            shared = len({o % 16 for o in offs + [d_off]}) == 1 and (contig or (ld * es) % 16 == 0)
            if flags & B.PTORED_LDS_PINGPONG and not shared and n > 1:
                assert B.PATHS[info.path] == "elementwise", label
            else:
                assert B.PATHS[info.path] != "elementwise", label
                if not shared and (contig or (ld * es) % 16 == 0):
                    origin = next(a for a in (1024, 128, 16) if contig or (ld * es) % a == 0)
                    assert info.lead == d_off % origin, label
                elif not shared:
                    assert info.lead == 0, label  # slots from each row's start
            dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc, offsets=offs,
                                    dst_offset=dst_off, tuning=t, alias=alias, label=label)
            assert st == 0, B.ptored_status_string(st)
            _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, alias=alias,
                   label=label)
            case += 1


@pytest.mark.parametrize("dtype", DT)
def test_row_tiles_with_spill_slots(dtype):
    """Row tiles whose rows end a few slots past their last whole tile: those
    slots folded in the tail tiles, one per lane across rows.  Reduction and
    allreduce, unrolled, two-slot (N <= 2) and runtime rank loops, and the
    LDS ping-pong variant."""
    rng = np.random.default_rng({"f32": 81, "bf16": 82, "f16": 83, "i32": 84}[dtype])
    es = ESIZE[dtype]
    for case, (rows, cols, ld, vr, vc, off) in enumerate(SPILL_SHAPES):
        if vc > cols:
            continue
        for n, flags in ((2, 0), (5, B.PTORED_ROW_TILES | B.PTORED_FORCE_ROWS),
                         (17, B.PTORED_FORCE_ROWS), (6, B.PTORED_LDS_PINGPONG)):
            if rows * ld * n > 30_000_000:
                continue
            root = int(rng.integers(0, n))
            op = OPS[(case + n) % 4]
            size = (rows - 1) * ld + cols
            srcs = [_rand_elems(dtype, rng, size) for _ in range(n)]
            t = B.tuning(flags=flags)
            label = f"spill#{case} N={n} {rows}x{cols} ld={ld} valid={vr}x{vc} off={off}"
            o = off - off % es
            dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc,
                                    offsets=[o] * n, dst_offset=o, tuning=t, label=label)
            assert st == 0, B.ptored_status_string(st)
            _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, label=label)
            # the in-place allreduce on the same buffers
            st = B.ptored_allreduce([b.ptr for b in bufs], n, root, rows, cols, ld, vr, vc,
                                    B.DTYPES[dtype], B.OPS[op], t,
                                    torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            assert st == 0, B.ptored_status_string(st)
            want = [x[:size].copy() for x in srcs]
            oracle.allreduce_inplace(want, root=root, dtype=dtype, op=op, rows=rows, cols=cols,
                                     ld=ld, valid_rows=vr, valid_cols=vc)
            for r, b in enumerate(bufs):
                assert compare(dtype, b.download(dtype), want[r]).all(), (label, "allreduce", r)
                assert b.guards_intact(), (label, r)


MEDIUM = [
    # rows, cols, ld, valid_rows, valid_cols
    (129, 1000, 1024, 129, 999),
    (3, 70001, 70008, 3, 70001),
    (64, 512, 512, 64, 512),
    (1, 200003, 200003, 1, 200003),
    (257, 333, 336, 250, 331),
    (60, 8200, 8200, 60, 8193),   # row tiles: 8 (f32) / 4 (16-bit) chunks per row + remainder
]


@pytest.mark.parametrize("dtype", DT)
def test_medium_cases_span_many_tiles(dtype):
    """Shapes that span many tiles and several grid-stride passes, with ragged
    row ends, one very long row and sub-rectangles."""
    rng = np.random.default_rng({"f32": 21, "bf16": 22, "f16": 23, "i32": 24}[dtype])
    for case, (rows, cols, ld, vr, vc) in enumerate(MEDIUM):
        for n, op, vname, flags, bpc in [(4, OPS[case % 4], "auto", 0, 1),
                                         (9, OPS[(case + 1) % 4], "flat",
                                          B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK, 0),
                                         (7, OPS[(case + 2) % 4], "full_occupancy",
                                          B.PTORED_FULL_OCCUPANCY, 0),
                                         (6, OPS[(case + 1) % 4], "row_tiles",
                                          B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES, 0),
                                         (11, OPS[(case + 2) % 4], "lds_pingpong",
                                          B.PTORED_LDS_PINGPONG, 0),
                                         (2, OPS[(case + 3) % 4], "lds_pingpong_n2",
                                          B.PTORED_LDS_PINGPONG, 1),
                                         (16, OPS[(case + 2) % 4], "auto", 0, 0),
                                         (20, OPS[(case + 3) % 4], "runtime_n", 0, 0),
                                         (3, OPS[case % 4], "elementwise",
                                          B.PTORED_FORCE_ELEMENTWISE, 2)]:
            size = (rows - 1) * ld + cols
            srcs = [_rand_elems(dtype, rng, size, wild=0.02) for _ in range(n)]
            root = int(rng.integers(0, n))
            t = B.tuning(flags=flags, blocks_per_cu=bpc)
            label = f"medium#{case} N={n} {vname}"
            dst, st, bufs = run_gpu(srcs, dtype, op, root, rows, cols, ld, vr, vc, tuning=t,
                                    label=label)
            assert st == 0
            _check(srcs, dtype, op, root, rows, cols, ld, vr, vc, dst, bufs, label=label)


@pytest.mark.parametrize("dtype", DT)
def test_split_into_many_launches(dtype):
    """A tiny launch byte limit splits one call into many launches: contiguous
    spans, row bands, and rows cut into spans."""
    rng = np.random.default_rng(31)
    es = ESIZE[dtype]
    for rows, cols, ld, vr, vc, mlb in [(40, 256, 256, 40, 256, 1024),
                                        (40, 250, 264, 37, 249, 3000),
                                        (5, 3000, 3008, 5, 2999, 512),
                                        (12, 4100, 4104, 12, 4099, 40000)]:
        n = 5
        size = (rows - 1) * ld + cols
        srcs = [_rand_elems(dtype, rng, size, wild=0.02) for _ in range(n)]
        for flags in (0, B.PTORED_FORCE_ELEMENTWISE, B.PTORED_ROW_TILES, B.PTORED_FLAT_WALK):
            t = B.tuning(flags=flags, max_launch_bytes=mlb)
            st_plan, info = B.ptored_treduce_plan([0x100000] * n, n, 1, 0x900000, rows, cols, ld,
                                                  vr, vc, B.DTYPES[dtype], 0, t)
            assert st_plan == 0 and info.launches > 1
            label = f"split mlb={mlb} launches={info.launches} flags={flags}"
            dst, st, bufs = run_gpu(srcs, dtype, "sum", 1, rows, cols, ld, vr, vc, tuning=t,
                                    label=label)
            assert st == 0
            _check(srcs, dtype, "sum", 1, rows, cols, ld, vr, vc, dst, bufs, label=label)


@pytest.mark.parametrize("dtype", DT)
def test_in_place_into_one_source(dtype):
    """dst is exactly one of the sources (the allreduce's in-place store)."""
    rng = np.random.default_rng(41)
    rows, cols, ld, vr, vc = 33, 500, 512, 30, 497
    size = (rows - 1) * ld + cols
    for n, alias, op in [(4, 0, "sum"), (4, 2, "max"), (12, 11, "min"), (1, 0, "sum"),
                         (20, 5, "sum")]:
        srcs = [_rand_elems(dtype, rng, size, wild=0.02) for _ in range(n)]
        dst, st, bufs = run_gpu(srcs, dtype, op, n // 2, rows, cols, ld, vr, vc, alias=alias,
                                label=f"alias={alias}")
        assert st == 0
        _check(srcs, dtype, op, n // 2, rows, cols, ld, vr, vc, dst, bufs, alias=alias,
               label=f"alias={alias}")


@pytest.mark.parametrize("dtype", DT)
def test_poison_outside_valid_never_reaches_output(dtype):
    rng = np.random.default_rng(51)
    rows, cols, ld, vr, vc, n = 20, 300, 304, 17, 293, 6
    size = (rows - 1) * ld + cols
    poison = {"f32": np.float32(np.nan), "i32": np.int32(-2**31), "bf16": np.uint16(0x7FC1),
              "f16": np.uint16(0x7E01)}[dtype]
    m = valid_mask(rows, ld, vr, vc, size)
    clean = [_rand_elems(dtype, rng, size, wild=0.0) for _ in range(n)]
    dirty = [np.where(m, s, poison).astype(s.dtype) for s in clean]
    for op in OPS:
        dst, st, bufs = run_gpu(dirty, dtype, op, 2, rows, cols, ld, vr, vc, label="poison")
        assert st == 0
        _check(dirty, dtype, op, 2, rows, cols, ld, vr, vc, dst, bufs, label="poison")
        want = oracle_reduce(clean, dtype, op, 2, rows, cols, ld, vr, vc,
                             lambda k: sentinel(dtype, k))
        assert compare(dtype, dst.download(dtype)[m], want[m]).all()


def test_rounding_edges_bf16_f16():
    """Operand pairs around ties, overflow and subnormals for the 16-bit float
    sums and products, every pattern against the oracle."""
    rng = np.random.default_rng(61)
    for dtype in ("bf16", "f16"):
        base = np.arange(0, 65536, dtype=np.uint32)
        near = (base + rng.integers(-4, 5, base.size)) & 0xFFFF
        far = rng.integers(0, 65536, base.size)
        a = np.concatenate([base, base]).astype(np.uint16)
        b = np.concatenate([near, far]).astype(np.uint16)
        for op in ("sum", "prod", "max", "min"):
            dst, st, bufs = run_gpu([a, b], dtype, op, 0, 1, a.size, a.size, 1, a.size,
                                    label="edges")
            assert st == 0
            _check([a, b], dtype, op, 0, 1, a.size, a.size, 1, a.size, dst, bufs,
                   label=f"edges {dtype} {op}")


def test_empty_region_launches_nothing_and_writes_nothing():
    d = DevBuf(1024)
    s = DevBuf(1024, fill=0)
    for vr, vc in ((0, 16), (16, 0)):
        st = B.ptored_treduce([s.ptr, s.ptr], 2, 0, d.ptr, 16, 16, 16, vr, vc, 0, 0,
                              torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == 0
        assert np.all(d.download_all() == 0xFF)


@pytest.mark.parametrize("dtype", DT)
def test_single_rank_is_a_bitwise_copy(dtype):
    """N == 1 copies the bits unchanged ([TREDUCE] §4.3 single-rank case):
    every 16-bit pattern (NaN payloads and signaling NaNs included) for the
    16-bit types, random 32-bit patterns plus signaling NaNs for f32 and i32;
    compared bit for bit, not by NaN-ness."""
    if ESIZE[dtype] == 2:
        src = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    else:
        rng = np.random.default_rng(5)
        src = rng.integers(0, 2 ** 32, 1 << 16, dtype=np.uint64).astype(np.uint32)
        src[:4] = [0x7F800001, 0xFF800001, 0x7FBFFFFF, 0x7FC00001]  # sNaNs, payload qNaN
    src = src.view(STORAGE[dtype])
    n = src.size
    for flags in (0, B.PTORED_FORCE_ELEMENTWISE):
        dst, st, bufs = run_gpu([src], dtype, "sum", 0, 1, n, n, 1, n,
                                tuning=B.tuning(flags=flags), label=f"copy flags={flags}")
        assert st == 0, B.ptored_status_string(st)
        got = dst.download(dtype)
        assert np.array_equal(got.view(np.uint8), src.view(np.uint8)), flags


def test_tensor_wrapper_and_side_stream():
    torch.manual_seed(0)
    xs = [torch.randn(300, 500, device="cuda") for _ in range(5)]
    out = torch.empty(300, 500, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        from cross_rank_collective_amd import treduce
        treduce(xs, out, op="max", root=3)
    s.synchronize()
    want = oracle_reduce([x.cpu().numpy().reshape(-1) for x in xs], "f32", "max", 3, 300, 500,
                         500, 300, 500, lambda k: sentinel("f32", k))
    assert np.array_equal(out.cpu().numpy().reshape(-1), want)
    with pytest.raises(B.PtoredError):
        treduce(xs, out, root=7)


# -------------------------------------------------- full-size workloads ---

def _workload_srcs(w):
    say("generate", w.name)
    return W.make_sources(w)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name):
    """Each named workload at its full size, in the launch configuration the
    benchmark uses and with every walk forced in turn: every valid element
    compared with the oracle (run in threaded row bands), and every byte
    outside the valid rectangle checked against the sentinel."""
    w = W.WORKLOADS[name]
    srcs = _workload_srcs(w)
    variants = [("auto", 0), ("row_tiles", B.PTORED_FORCE_ROWS | B.PTORED_ROW_TILES),
                ("flat", B.PTORED_FORCE_ROWS | B.PTORED_FLAT_WALK),
                ("lds_pingpong", B.PTORED_LDS_PINGPONG)]
    es = w.esize
    m = valid_mask(w.rows, w.ld, w.valid_rows, w.valid_cols, w.buffer_elems)
    for op in w.ops:
        say(name, op, "oracle (row bands)")
        want = oracle_reduce_banded(srcs, w.dtype, op, w.root, w.rows, w.cols, w.ld,
                                    w.valid_rows, w.valid_cols)
        want_valid = want[m]
        del want
        for vname, flags in variants:
            label = f"{name} {op} {vname}"
            dst, st, bufs = run_gpu(srcs, w.dtype, op, w.root, w.rows, w.cols, w.ld,
                                    w.valid_rows, w.valid_cols, tuning=B.tuning(flags=flags),
                                    label=label)
            assert st == 0
            del bufs
            got = dst.download(w.dtype)
            assert dst.guards_intact()
            # untouched outside the valid rectangle, over the whole buffer
            assert np.all(got.view(np.uint8).reshape(-1, es)[~m] == 0xFF), label
            ok = compare(w.dtype, got[m], want_valid)
            assert ok.all(), (label, int((~ok).sum()), int(np.argmin(ok)))
            del got, dst
        torch.cuda.empty_cache()
