"""CPU oracle for the N-way TREDUCE reduction -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product library and its Python
binding never import, load or call it, and it shares no code with them.

The arithmetic lives in ``treduce_oracle.c`` (plain loops, one element at a
time, in the order of "CANN PTO-ISA TREDUCE instruction explained" §4.3);
this module compiles it with gcc and marshals numpy arrays into it.

Element buffers are passed as numpy arrays of the raw element bits:
``float32`` for f32, ``int32`` for i32, ``uint16`` for bf16 and f16.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "treduce_oracle.c")
_LIB = os.path.join(_HERE, "libtreduce_oracle.so")
# A separately built copy of the same source (the sanitizer run builds one
# with -fsanitize=address,undefined) may be named here; it is loaded as is.
_LIB_OVERRIDE = os.environ.get("PTORED_ORACLE_LIB")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3}
OPS = {"sum": 0, "max": 1, "min": 2, "prod": 3}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "i32": np.int32}

_lib = None


def build(out: str = _LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the oracle with gcc (IEEE arithmetic: no contraction, no fast-math)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fno-finite-math-only", "-Wall", "-Wextra", "-shared", "-fPIC", *extra_flags,
        "-o", out + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_treduce.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, vp,
                                   i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_treduce.restype = ctypes.c_int
    lib.oracle_allreduce_inplace.argtypes = [ctypes.POINTER(vp), ctypes.c_int, ctypes.c_int, vp,
                                             i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int]
    lib.oracle_allreduce_inplace.restype = ctypes.c_int
    lib.oracle_combine_bits.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, i64]
    lib.oracle_combine_bits.restype = None
    lib.oracle_round_from_double.argtypes = [ctypes.c_int, vp, vp, i64]
    lib.oracle_round_from_double.restype = None
    lib.oracle_to_double.argtypes = [ctypes.c_int, vp, vp, i64]
    lib.oracle_to_double.restype = None
    lib.oracle_max_ranks.restype = ctypes.c_int
    lib.oracle_ring_bounds.argtypes = [i64, ctypes.c_int, ctypes.c_int, vp]
    lib.oracle_ring_bounds.restype = ctypes.c_int
    lib.oracle_reduce_scatter_ring.argtypes = [ctypes.POINTER(vp), ctypes.c_int,
                                               ctypes.POINTER(vp), i64, ctypes.c_int,
                                               ctypes.c_int]
    lib.oracle_reduce_scatter_ring.restype = ctypes.c_int
    lib.oracle_accumulate_add.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, i64, i64, i64,
                                          i64, i64, ctypes.c_int, vp, vp]
    lib.oracle_accumulate_add.restype = ctypes.c_int
    _lib = lib
    return lib


def _check_buffers(arrs: Sequence[np.ndarray], dtype: str, rows: int, ld: int, cols: int):
    need = (rows - 1) * ld + cols if rows > 0 else 0
    for a in arrs:
        if a.dtype != STORAGE[dtype]:
            raise TypeError(f"oracle buffer dtype {a.dtype} does not hold {dtype}")
        if not a.flags.c_contiguous:
            raise ValueError("oracle buffers must be C-contiguous")
        if a.size < need:
            raise ValueError(f"oracle buffer of {a.size} elements is smaller than {need}")


def treduce(srcs: Sequence[np.ndarray], dst: np.ndarray, *, root: int, dtype: str, op: str,
            rows: int, cols: int, ld: int, valid_rows: int, valid_cols: int) -> None:
    """dst[i*ld+j] = (+)_r srcs[r][i*ld+j] over the valid rectangle, in place in ``dst``."""
    lib = _load()
    _check_buffers(list(srcs) + [dst], dtype, rows, ld, cols)
    ptrs = (ctypes.c_void_p * max(1, len(srcs)))(*[a.ctypes.data for a in srcs])
    rc = lib.oracle_treduce(ptrs, len(srcs), root, dst.ctypes.data, rows, cols, ld,
                            valid_rows, valid_cols, DTYPES[dtype], OPS[op])
    if rc != 0:
        raise ValueError(f"oracle_treduce rejected its arguments (status {rc})")


def treduce_banded(srcs: Sequence[np.ndarray], dst: np.ndarray, *, root: int, dtype: str,
                   op: str, rows: int, cols: int, ld: int, valid_rows: int, valid_cols: int,
                   threads: int = 8) -> None:
    """``treduce`` over large buffers: the valid rows are cut into `threads`
    contiguous bands and each band is one ``treduce`` call on its own thread
    (the C code runs without the GIL).  Every element is still computed by
    the same plain loop; bands only partition independent elements."""
    from concurrent.futures import ThreadPoolExecutor

    _check_buffers(list(srcs) + [dst], dtype, rows, ld, cols)
    if valid_rows == 0 or valid_cols == 0 or threads <= 1 or valid_rows < 2 * threads:
        treduce(srcs, dst, root=root, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                valid_rows=valid_rows, valid_cols=valid_cols)
        return
    cuts = [valid_rows * k // threads for k in range(threads + 1)]

    def band(k):
        r0, r1 = cuts[k], cuts[k + 1]
        off = r0 * ld
        size = (r1 - r0 - 1) * ld + cols
        treduce([s[off:off + size] for s in srcs], dst[off:off + size], root=root,
                dtype=dtype, op=op, rows=r1 - r0, cols=cols, ld=ld, valid_rows=r1 - r0,
                valid_cols=valid_cols)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(band, range(threads)))


def allreduce_inplace(bufs: Sequence[np.ndarray], *, root: int, dtype: str, op: str, rows: int,
                      cols: int, ld: int, valid_rows: int, valid_cols: int) -> None:
    """Reduce all buffers and write the result back into every one of them."""
    lib = _load()
    _check_buffers(bufs, dtype, rows, ld, cols)
    scratch = np.zeros_like(bufs[0])
    ptrs = (ctypes.c_void_p * len(bufs))(*[a.ctypes.data for a in bufs])
    rc = lib.oracle_allreduce_inplace(ptrs, len(bufs), root, scratch.ctypes.data, rows, cols,
                                      ld, valid_rows, valid_cols, DTYPES[dtype], OPS[op])
    if rc != 0:
        raise ValueError(f"oracle_allreduce_inplace rejected its arguments (status {rc})")


def ring_bounds(count: int, nranks: int, dtype: str) -> np.ndarray:
    """Segment boundaries (nranks + 1 of them) of the ring schedule."""
    lib = _load()
    out = np.zeros(nranks + 1, dtype=np.int64)
    rc = lib.oracle_ring_bounds(count, nranks, DTYPES[dtype], out.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_ring_bounds rejected its arguments (status {rc})")
    return out


def reduce_scatter_ring(srcs: Sequence[np.ndarray], dsts: Sequence[np.ndarray], *, count: int,
                        dtype: str, op: str) -> None:
    """dsts[s][segment s] = ring-order fold of every source over segment s."""
    lib = _load()
    _check_buffers(list(srcs) + list(dsts), dtype, 1, count, count)
    sp = (ctypes.c_void_p * len(srcs))(*[a.ctypes.data for a in srcs])
    dp = (ctypes.c_void_p * len(dsts))(*[a.ctypes.data for a in dsts])
    rc = lib.oracle_reduce_scatter_ring(sp, len(srcs), dp, count, DTYPES[dtype], OPS[op])
    if rc != 0:
        raise ValueError(f"oracle_reduce_scatter_ring rejected its arguments (status {rc})")


def accumulate_add(srcs: Sequence[np.ndarray], dst: np.ndarray, *, dtype: str, rows: int,
                   cols: int, ld: int, valid_rows: int, valid_cols: int):
    """dst += every source, in rank order with element rounding; returns the
    exact sums and the absolute sums over the valid rectangle (float types)."""
    lib = _load()
    _check_buffers(list(srcs) + [dst], dtype, rows, ld, cols)
    ptrs = (ctypes.c_void_p * max(1, len(srcs)))(*[a.ctypes.data for a in srcs])
    exact = np.zeros(valid_rows * valid_cols, dtype=np.float64)
    absum = np.zeros(valid_rows * valid_cols, dtype=np.float64)
    rc = lib.oracle_accumulate_add(ptrs, len(srcs), dst.ctypes.data, rows, cols, ld, valid_rows,
                                   valid_cols, DTYPES[dtype], exact.ctypes.data,
                                   absum.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_accumulate_add rejected its arguments (status {rc})")
    return exact, absum


def combine_bits(dtype: str, op: str, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """One combine step on raw element bits held in uint32 arrays."""
    lib = _load()
    a = np.ascontiguousarray(a, dtype=np.uint32)
    b = np.ascontiguousarray(b, dtype=np.uint32)
    out = np.empty_like(a)
    lib.oracle_combine_bits(DTYPES[dtype], OPS[op], a.ctypes.data, b.ctypes.data,
                            out.ctypes.data, a.size)
    return out


def round_from_double(dtype: str, x: np.ndarray) -> np.ndarray:
    """Nearest element of a float dtype to each double, ties to even; uint32 bits."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint32)
    lib.oracle_round_from_double(DTYPES[dtype], x.ctypes.data, out.ctypes.data, x.size)
    return out


def to_double(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Exact value of each element's bits (uint32 holding the element)."""
    lib = _load()
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_to_double(DTYPES[dtype], bits.ctypes.data, out.ctypes.data, bits.size)
    return out


def max_ranks() -> int:
    return int(_load().oracle_max_ranks())
