"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, maps one HIP runtime, and returns every error status (and the empty
short-circuit) before it makes any HIP call."""

import os
import re

import pytest

import cross_rank_collective_amd as crc
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Fake device addresses: never dereferenced, because every call below stops
# in the host-side checks or the empty short-circuit.
A = [0x10000000 + 0x1000000 * r for r in range(80)]
D = 0x7F000000


def _header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ptored_\w+)\s*\(", text,
                                    flags=re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _header_functions()
    for n in ("ptored_treduce", "ptored_treduce_ex", "ptored_treduce_plan",
              "ptored_status_string", "ptored_abi_version", "ptored_max_ranks"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_one_hip_runtime_is_mapped():
    B.load()
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths


def test_version_and_limits():
    assert crc.ptored_abi_version() == 3
    assert crc.ptored_max_ranks() == 64


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        s = crc.ptored_status_string(st)
        assert s.startswith("PTORED_")
    assert "unknown" in crc.ptored_status_string(7)


def _call(n=2, root=0, dst=D, rows=4, cols=4, ld=4, vr=4, vc=4, dtype=0, op=0, srcs=None):
    srcs = A[:n] if srcs is None else srcs
    return crc.ptored_treduce(srcs, n, root, dst, rows, cols, ld, vr, vc, dtype, op, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), -1), (dict(n=65), -1), (dict(root=2), -1), (dict(root=-1), -1),
    (dict(dst=0), -1), (dict(srcs=[A[0], 0]), -1), (dict(rows=-1), -1), (dict(cols=-1), -1),
    (dict(ld=-1), -1), (dict(vr=-1), -1), (dict(vc=-1), -1), (dict(cols=5), -1),
    (dict(vr=5), -1), (dict(vc=5, cols=4, ld=8), -1), (dict(rows=1 << 40, ld=1 << 30), -1),
    (dict(dtype=4), -2), (dict(dtype=-1), -2), (dict(op=4), -2), (dict(op=-1), -2),
    (dict(dst=A[1] + 4), -3), (dict(dst=A[0] - 8), -3),
    (dict(dst=D + 2), -1), (dict(srcs=[A[0], A[1] + 1]), -1), (dict(dst=D + 1, dtype=2), -1),
])
def test_argument_errors_before_any_hip_call(kw, status):
    assert _call(**kw) == status


def test_invalid_beats_unsupported_beats_overlap():
    assert _call(root=9, dtype=9) == -1
    assert _call(dtype=9, dst=A[1] + 4) == -2
    assert _call(dst=A[1] + 2) == -1  # misaligned element pointer before overlap


def test_empty_region_returns_ok_without_launch():
    assert _call(vr=0) == 0
    assert _call(vc=0) == 0
    assert _call(rows=0, vr=0) == 0
    assert _call(n=64, srcs=A[:64], vr=0, dtype=2, op=3) == 0


def _plan(n=2, root=0, dst=D, rows=4, cols=4, ld=4, vr=4, vc=4, dtype=0, op=0, srcs=None,
          tuning=None):
    srcs = A[:n] if srcs is None else srcs
    st, info = crc.ptored_treduce_plan(srcs, n, root, dst, rows, cols, ld, vr, vc, dtype, op,
                                       tuning)
    assert st == 0
    return info


def test_exact_alias_is_allowed_in_place():
    info = _plan(n=3, dst=A[1])
    assert B.PATHS[info.path] == "vec_fixed"


def test_plan_paths():
    assert B.PATHS[_plan(vr=0).path] == "none"
    assert B.PATHS[_plan(n=1).path] == "copy"
    assert B.PATHS[_plan(n=16, srcs=A[:16]).path] == "vec_fixed"
    assert B.PATHS[_plan(n=17, srcs=A[:17]).path] == "vec_runtime"
    assert B.PATHS[_plan(n=64, srcs=A[:64]).path] == "vec_runtime"
    # buffers at different offsets within 16 bytes, or a row pitch off the
    # 16-byte grid, keep the vector path with unaligned accesses ...
    assert B.PATHS[_plan(srcs=[A[0], A[1] + 4]).path] == "vec_fixed"
    assert B.PATHS[_plan(dst=D + 2, dtype=2).path] == "vec_fixed"
    assert B.PATHS[_plan(rows=4, cols=3, ld=5, vr=4, vc=3).path] == "vec_fixed"
    # ... except through the LDS variant, which keeps the shared-offset rule
    t = B.tuning(flags=B.PTORED_LDS_PINGPONG)
    assert B.PATHS[_plan(n=5, srcs=A[:4] + [A[4] + 4], tuning=t).path] == "elementwise"
    assert B.PATHS[_plan(n=5, srcs=A[:5], tuning=t, rows=4, cols=3, ld=5, vr=4,
                         vc=3).path] == "elementwise"
    # forcing flags
    t = B.tuning(flags=B.PTORED_FORCE_ELEMENTWISE)
    assert B.PATHS[_plan(tuning=t).path] == "elementwise"
    t = B.tuning(flags=B.PTORED_FORCE_RUNTIME_N)
    assert B.PATHS[_plan(tuning=t).path] == "vec_runtime"
    t = B.tuning(flags=B.PTORED_LDS_PINGPONG)
    info = _plan(n=5, srcs=A[:5], tuning=t)
    assert (B.PATHS[info.path], info.slots_per_thread) == ("vec_runtime", 1)
    assert B.PATHS[_plan(n=1, tuning=t).path] == "copy"  # one rank: nothing to stage


def test_plan_resident_workgroups():
    """Workgroups (one wave each) kept resident per CU by one-tile-per-block
    launches, by rank count: 16 up to 3 ranks, 12 at 4-5, 10 at 6-7, 8 from
    8 on, 6 from 12 on for 4-byte types; 10 for the runtime rank loop; no
    limit for the element-wise kernel, persistent grids or on request."""
    assert _plan(n=16, srcs=A[:16], dtype=3).wgs_per_cu == 6
    assert _plan(n=16, srcs=A[:16], dtype=1).wgs_per_cu == 8
    assert _plan(n=8, srcs=A[:8], dtype=1).wgs_per_cu == 8
    assert _plan(n=11, srcs=A[:11]).wgs_per_cu == 8
    assert _plan(n=12, srcs=A[:12]).wgs_per_cu == 6
    assert _plan(n=12, srcs=A[:12], dtype=2).wgs_per_cu == 8
    assert _plan(n=6, srcs=A[:6]).wgs_per_cu == 10
    assert _plan(n=5, srcs=A[:5]).wgs_per_cu == 12
    assert _plan(n=4, srcs=A[:4]).wgs_per_cu == 12
    assert _plan(n=2, srcs=A[:2]).wgs_per_cu == 16
    assert _plan(n=1).wgs_per_cu == 16                         # copy
    assert _plan(n=17, srcs=A[:17]).wgs_per_cu == 10           # runtime rank loop
    info = _plan(n=64, srcs=A[:64])
    assert (info.wgs_per_cu, info.slots_per_thread) == (10, 1)
    assert _plan(srcs=[A[0], A[1] + 4]).wgs_per_cu == 16       # unaligned: same rule
    t = B.tuning(flags=B.PTORED_FORCE_ELEMENTWISE)
    assert _plan(tuning=t).wgs_per_cu == 0                     # element-wise
    assert _plan(tuning=B.tuning(flags=B.PTORED_FULL_OCCUPANCY)).wgs_per_cu == 0
    assert _plan(tuning=B.tuning(blocks_per_cu=2)).wgs_per_cu == 0
    assert _plan(vr=0).wgs_per_cu == 0


def test_plan_common_lead():
    """Buffers that all start the same number of bytes past a 16-byte boundary
    keep the vector path (rows begin with a head); buffers at different
    offsets take dst's alignment (the sources are read unaligned), a pitch
    off the 16-byte grid numbers each row's slots from its start, and a row
    too short to reach the boundary selects the element-wise kernel."""
    co = [A[0] + 4, A[1] + 4]
    info = _plan(srcs=co, dst=D + 4)                               # 16 contiguous f32
    assert (B.PATHS[info.path], info.lead, info.launches) == ("vec_fixed", 4, 1)
    info = _plan(srcs=co, dst=D + 8)                               # dst at another offset
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 8)
    info = _plan(srcs=co, dst=D + 520)                             # dst's 1 KiB offset
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 520)
    info = _plan(srcs=[A[0] + 6, A[1] + 6], dst=D + 6, dtype=2, rows=8, cols=10, ld=16,
                 vr=7, vc=9)                                       # f16 rows of 32 B pitch
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 6)
    info = _plan(srcs=[A[0] + 6, A[1] + 10], dst=D + 2, dtype=2, rows=8, cols=10, ld=16,
                 vr=7, vc=9)                                       # dst's offset, 32 B pitch
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 2)
    info = _plan(srcs=[A[0] + 6, A[1] + 6], dst=D + 6, dtype=2, rows=8, cols=10, ld=12,
                 vr=7, vc=9)                                       # 24 B pitch: row starts
    assert (B.PATHS[info.path], info.rows_mode != 0, info.lead) == ("vec_fixed", True, 0)
    info = _plan(srcs=[A[0] + 12, A[1] + 12], dst=D + 12, rows=1, cols=1, ld=1, vr=1, vc=1)
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 12)   # exactly [12, 16)
    info = _plan(srcs=[A[0] + 8, A[1] + 8], dst=D + 8, rows=1, cols=1, ld=1, vr=1, vc=1)
    assert B.PATHS[info.path] == "elementwise"                     # [8, 12) never reaches 16
    # windows stay on the 16-byte grid: 4 + 64 bytes in windows of 32
    info = _plan(srcs=co, dst=D + 4, tuning=B.tuning(max_launch_bytes=32))
    assert info.launches == 3


def test_plan_line_origin():
    """Slots are numbered from the coarsest of a 1 KiB, 128-byte or 16-byte
    boundary at which every buffer (and, for rows, the pitch) has the same
    offset; lead = that offset, with heads when it is inside a 16-byte block."""
    info = _plan(srcs=[A[0] + 16, A[1] + 144], dst=D + 400)        # 16 mod 128
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 16)
    info = _plan(srcs=[A[0] + 100, A[1] + 100], dst=D + 100)       # 100 mod 128: a head
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 100)
    info = _plan(srcs=[A[0] + 16, A[1] + 32], dst=D + 16)          # only 0 mod 16 in common
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 0)
    info = _plan(srcs=[A[0] + 36, A[1] + 52], dst=D + 4)           # only 4 mod 16
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 4)
    # 2-D: a pitch of 512 bytes keeps the line offset, one of 48 bytes does not
    info = _plan(srcs=[A[0] + 36, A[1] + 36], dst=D + 36, rows=8, cols=100, ld=128, vr=8,
                 vc=100)
    assert (B.PATHS[info.path], info.rows_mode != 0, info.lead) == ("vec_fixed", True, 36)
    info = _plan(srcs=[A[0] + 36, A[1] + 36], dst=D + 36, rows=8, cols=10, ld=12, vr=8, vc=10)
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 4)
    info = _plan(srcs=[A[0] + 528, A[1] + 1552], dst=D + 528)      # 528 mod 1024
    assert (B.PATHS[info.path], info.lead) == ("vec_fixed", 528)
    info = _plan(srcs=[A[0] + 528, A[1] + 528], dst=D + 528, rows=8, cols=256, ld=256, vr=8,
                 vc=250)                                           # 1 KiB pitch keeps it
    assert (info.rows_mode != 0, info.lead) == (True, 528)
    info = _plan(srcs=[A[0] + 528, A[1] + 528], dst=D + 528, rows=8, cols=100, ld=128, vr=8,
                 vc=100)                                           # 512 B pitch: the line
    assert info.lead == 16
    # launch windows that lie wholly before the data are not launched: bytes
    # [100, 356) in windows of 32 meet windows 3 .. 11
    info = _plan(srcs=[A[0] + 100, A[1] + 100], dst=D + 100, rows=1, cols=64, ld=64, vr=1,
                 vc=64, tuning=B.tuning(max_launch_bytes=32))
    assert (info.lead, info.launches) == (100, 9)


def test_plan_walk_and_slots():
    info = _plan(rows=8, cols=8, ld=8, vr=8, vc=8)  # contiguous f32
    assert (info.rows_mode, info.vec_elems, info.slots, info.launches) == (0, 4, 16, 1)
    info = _plan(rows=8, cols=10, ld=12, vr=7, vc=10)  # narrow rows: flattened, 3 slots/row
    assert (info.rows_mode, info.slots) == (2, 21)
    info = _plan(rows=8, cols=8, ld=8, vr=8, vc=8, tuning=B.tuning(flags=B.PTORED_FORCE_ROWS))
    assert (info.rows_mode, info.slots) == (2, 16)  # 2 slots per row fill 1/32 of a chunk
    # wide rows: row tiles (tile = row x column chunk of 64 slots) when a row's
    # slots fill its chunks: 1000 f32 = 250 slots in 4 chunks; flattened on request
    info = _plan(n=4, srcs=A[:4], rows=64, cols=1000, ld=1024, vr=60, vc=1000)
    assert (info.rows_mode, info.slots) == (1, 60 * 250)
    flat = B.tuning(flags=B.PTORED_FLAT_WALK)
    info = _plan(n=4, srcs=A[:4], rows=64, cols=1000, ld=1024, vr=60, vc=1000, tuning=flat)
    assert (info.rows_mode, info.slots) == (2, 60 * 250)
    # 100 slots: one whole chunk of 64 and a last one 36/64 full (more than half,
    # so it stays a tile): 100/128 of the threads busy -> flattened, unless row
    # tiles are forced
    info = _plan(n=4, srcs=A[:4], rows=4, cols=400, ld=404, vr=4, vc=400)
    assert info.rows_mode == 2
    rt = B.tuning(flags=B.PTORED_ROW_TILES)
    info = _plan(n=4, srcs=A[:4], rows=4, cols=400, ld=404, vr=4, vc=400, tuning=rt)
    assert info.rows_mode == 1
    # 65 slots: one whole chunk, the last slot of each row spills into the tail
    # tiles, so the row tiles are full -> row tiles
    info = _plan(n=4, srcs=A[:4], rows=4, cols=260, ld=264, vr=4, vc=260)
    assert info.rows_mode == 1
    # 8 or more chunks per row: row tiles whatever the last chunk holds
    info = _plan(n=4, srcs=A[:4], rows=4, cols=4 * 7 * 64 + 4, ld=1800, vr=4, vc=1796)
    assert info.rows_mode == 1
    # the LDS variant takes the same walks
    lds = B.tuning(flags=B.PTORED_LDS_PINGPONG)
    info = _plan(n=4, srcs=A[:4], rows=64, cols=1000, ld=1024, vr=60, vc=1000, tuning=lds)
    assert info.rows_mode == 1
    info = _plan(n=4, srcs=A[:4], rows=64, cols=1000, ld=1024, vr=60, vc=1000,
                 tuning=B.tuning(flags=B.PTORED_LDS_PINGPONG | B.PTORED_FLAT_WALK))
    assert info.rows_mode == 2
    info = _plan(rows=1, cols=13, ld=16, vr=1, vc=13, dtype=2)  # one row: contiguous f16
    assert (info.rows_mode, info.vec_elems, info.slots) == (0, 8, 2)


def test_plan_launch_split():
    # contiguous: 4096 f32 = 16 KiB in launches of 4 KiB
    info = _plan(rows=64, cols=64, ld=64, vr=64, vc=64, tuning=B.tuning(max_launch_bytes=4096))
    assert info.launches == 4
    # rows: 10 rows, pitch 64 B, 40 valid bytes per row, 256-byte launches:
    # (256 - 40) // 64 + 1 = 4 rows per launch -> 3 launches
    info = _plan(rows=10, cols=10, ld=16, vr=10, vc=10, tuning=B.tuning(max_launch_bytes=256))
    assert (info.rows_mode, info.launches) == (2, 3)
    # rows longer than one launch: every row is split into spans
    info = _plan(rows=3, cols=100, ld=104, vr=3, vc=100, tuning=B.tuning(max_launch_bytes=128))
    assert info.launches == 3 * 4


def test_workload_plans():
    """Each named workload takes the kernel family its shape calls for."""
    want = {
        "n2_f32_16x16": ("vec_fixed", 0),
        "n4_f32_1024x1024_valid1000x1000": ("vec_fixed", 1),
        "n8_bf16_8192x8192": ("vec_fixed", 0),
        "n16_i32_4096x4096": ("vec_fixed", 0),
        "n8_f16_8192x12288_valid8191x12287": ("vec_fixed", 1),
    }
    for name, w in W.WORKLOADS.items():
        info = _plan(n=w.nranks, srcs=A[:w.nranks], rows=w.rows, cols=w.cols, ld=w.ld,
                     vr=w.valid_rows, vc=w.valid_cols, dtype=B.DTYPES[w.dtype],
                     op=B.OPS[w.ops[0]])
        assert (B.PATHS[info.path], info.rows_mode) == want[name], name  # 1 = row tiles
        assert info.launches == 1


def test_ring_bounds_match_the_oracle_rule():
    import oracle
    rng = __import__("numpy").random.default_rng(4)
    for _ in range(200):
        count = int(rng.integers(0, 100000))
        n = int(rng.integers(1, 65))
        for dt, code in B.DTYPES.items():
            st, b = crc.ptored_ring_bounds(count, n, code)
            assert st == 0
            assert b == list(oracle.ring_bounds(count, n, dt))
    assert crc.ptored_ring_bounds(10, 0, 0)[0] == -1
    assert crc.ptored_ring_bounds(-1, 2, 0)[0] == -1
    assert crc.ptored_ring_bounds(10, 2, 7)[0] == -2


def test_collective_argument_errors_before_any_hip_call():
    lib = B
    s = 0
    # allreduce: bad root, partial overlap between buffers, misaligned pointer
    assert lib.ptored_allreduce(A[:2], 2, 2, 4, 4, 4, 4, 4, 0, 0, None, s) == -1
    assert lib.ptored_allreduce([A[0], A[0] + 8], 2, 0, 4, 4, 4, 4, 4, 0, 0, None, s) == -3
    assert lib.ptored_allreduce([A[0], A[1] + 2], 2, 0, 4, 4, 4, 4, 4, 0, 0, None, s) == -1
    assert lib.ptored_allreduce(A[:2], 2, 0, 4, 4, 4, 0, 4, 0, 0, None, s) == 0  # empty
    assert lib.ptored_allreduce([A[0]], 1, 0, 4, 4, 4, 4, 4, 0, 0, None, s) == 0  # N == 1
    # reduce-scatter: partial overlap of a dst with a source, bad op, empty stream
    assert lib.ptored_reduce_scatter_ring(A[:2], 2, [A[2], A[0] + 16], 64, 0, 0, None, s) == -3
    assert lib.ptored_reduce_scatter_ring(A[:2], 2, A[2:4], 64, 0, 9, None, s) == -2
    assert lib.ptored_reduce_scatter_ring(A[:2], 2, A[2:4], 0, 0, 0, None, s) == 0
    assert lib.ptored_reduce_scatter_ring(A[:2], 2, A[2:4], -1, 0, 0, None, s) == -1
    # accumulate: dst may not alias a source, even exactly
    assert lib.ptored_accumulate_add(A[:2], 2, A[1], 4, 4, 4, 4, 4, 0, None, s) == -3
    assert lib.ptored_accumulate_add(A[:2], 2, D, 4, 4, 4, 0, 4, 0, None, s) == 0  # empty


def test_header_as_c11_against_the_library(tmp_path):
    """include/ptored.h compiled as C11 (gcc, warnings as errors) and linked
    with the built library: layouts, enum values, plans, argument errors and
    ring bounds checked from C (tests/c_abi_check.c); no HIP call is made."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    libdir = os.path.join(root, "cross_rank_collective_amd")
    exe = str(tmp_path / "c_abi_check")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(root, "include"), "-I/opt/rocm/include",
           os.path.join(here, "c_abi_check.c"), "-L" + libdir, "-lptored",
           "-Wl,-rpath," + libdir, "-o", exe]
    subprocess.run(cmd, check=True)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0 and "c abi ok" in out.stdout, out.stdout + out.stderr


def test_tensor_wrappers_reject_bad_groups():
    """The tensor wrappers check their arguments before calling the library."""
    import torch

    import cross_rank_collective_amd as crc

    a = torch.zeros(4, 8)
    with pytest.raises(ValueError):
        crc.allreduce([])
    with pytest.raises(ValueError):
        crc.reduce_scatter_ring([a], [])
    with pytest.raises(ValueError):
        crc.accumulate_add([], a)
    with pytest.raises(TypeError):
        crc.ring_bounds(10, 2, torch.float64)
    with pytest.raises(ValueError):  # CPU tensors are not on a GPU
        crc.allreduce([a, torch.zeros(4, 8)])
    assert crc.ring_bounds(100, 4, "bf16") == [0, 32, 64, 80, 100]
    with pytest.raises(ValueError):  # an op the library does not have
        crc.treduce([a, a], torch.zeros(4, 8), op="mean")


def test_c_consumer_program_compiles(tmp_path):
    """The C program of the GPU test (tests/c_consumer_gpu.c) builds against the
    header, the library and the oracle with warnings as errors."""
    from tests.test_c_consumer_gpu import _build

    assert os.path.exists(_build(tmp_path))


def test_binding_constants_match_the_header():
    """Every numeric #define of include/ptored.h that the binding mirrors has
    the same value there (flags, limits, the workgroup size)."""
    import re

    here = os.path.dirname(os.path.abspath(__file__))
    text = open(os.path.join(os.path.dirname(here), "include", "ptored.h")).read()
    defines = dict(re.findall(r"^#define (PTORED_\w+) (0x[0-9a-fA-F]+|\d+)", text, re.M))
    assert "PTORED_WORKGROUP_THREADS" in defines and "PTORED_FLAT_WALK" in defines
    checked = 0
    for name, value in defines.items():
        if hasattr(B, name):
            assert getattr(B, name) == int(value.rstrip("uU"), 0), name
            checked += 1
    assert checked == 12  # ten flags, the rank limit and the workgroup size
    paths = {int(v): k[len("PTORED_PATH_"):].lower() for k, v in defines.items()
             if k.startswith("PTORED_PATH_")}
    assert paths == {0: "none", 1: "copy", 2: "vec_fixed", 3: "vec_runtime", 4: "elementwise"}
    assert B.PATHS == paths


def test_prebuilt_pointer_array_is_passed_as_is():
    """Raw calls take a prebuilt pointer array (built once for repeated calls)
    and plan it like the list it was built from."""
    arr = B.pointer_array(A[:4])
    assert B._ptrs(arr) is arr
    assert list(arr) == list(A[:4])
    st1, i1 = crc.ptored_treduce_plan(arr, 4, 0, D, 4, 4, 4, 4, 4, 0, 0)
    st2, i2 = crc.ptored_treduce_plan(A[:4], 4, 0, D, 4, 4, 4, 4, 4, 0, 0)
    assert st1 == st2 == 0
    assert (i1.path, i1.slots, i1.lead) == (i2.path, i2.slots, i2.lead)
