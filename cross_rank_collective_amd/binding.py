"""ctypes binding of libptored.so (argument marshalling only).

Every step of the reduction runs in the library's HIP kernels; this module
only turns Python values and torch tensors into the C ABI's pointers and
sizes.  torch provides device memory and the stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.

The C functions keep their names: ``ptored_treduce``, ``ptored_treduce_ex``,
``ptored_treduce_plan``, ``ptored_allreduce``, ``ptored_ring_bounds``,
``ptored_reduce_scatter_ring``, ``ptored_accumulate_add``,
``ptored_status_string``, ``ptored_abi_version``, ``ptored_max_ranks``.
``treduce`` is the tensor-level convenience wrapper.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libptored.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3}
OPS = {"sum": 0, "max": 1, "min": 2, "prod": 3}

PTORED_OK = 0
PTORED_ERR_INVALID_ARG = -1
PTORED_ERR_UNSUPPORTED = -2
PTORED_ERR_OVERLAP = -3
PTORED_ERR_HIP = -4

PTORED_FORCE_ELEMENTWISE = 0x1
PTORED_FORCE_ROWS = 0x2
PTORED_FORCE_RUNTIME_N = 0x4
PTORED_NO_XCD_REMAP = 0x8
PTORED_ROW_TILES = 0x10
PTORED_LDS_PINGPONG = 0x20
PTORED_SEGMENT_LAUNCHES = 0x40
PTORED_FULL_OCCUPANCY = 0x80
PTORED_FLAT_WALK = 0x100
PTORED_ACC_PER_RANK = 0x200

PTORED_MAX_RANKS = 64
PTORED_WORKGROUP_THREADS = 64  # threads per workgroup of the kernels (one wave)

PATHS = {0: "none", 1: "copy", 2: "vec_fixed", 3: "vec_runtime", 4: "elementwise"}


class ptored_tuning(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("blocks_per_cu", ctypes.c_int32),
                ("max_launch_bytes", ctypes.c_int64)]


class ptored_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("rows_mode", ctypes.c_int32),
                ("vec_elems", ctypes.c_int32), ("slots_per_thread", ctypes.c_int32),
                ("slots", ctypes.c_int64), ("launches", ctypes.c_int64),
                ("wgs_per_cu", ctypes.c_int32), ("lead", ctypes.c_int32)]


class PtoredError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libptored.so (after torch, so one HIP runtime serves both)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- maps torch's libamdhip64 first

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m cross_rank_collective_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    common = [ctypes.POINTER(vp), i32, i32, vp, i64, i64, i64, i64, i64, i32, i32]
    lib.ptored_treduce.argtypes = common + [vp]
    lib.ptored_treduce.restype = i32
    lib.ptored_treduce_ex.argtypes = common + [ctypes.POINTER(ptored_tuning), vp]
    lib.ptored_treduce_ex.restype = i32
    lib.ptored_treduce_plan.argtypes = common + [ctypes.POINTER(ptored_tuning),
                                                 ctypes.POINTER(ptored_plan_info)]
    lib.ptored_treduce_plan.restype = i32
    lib.ptored_allreduce.argtypes = [ctypes.POINTER(vp), i32, i32, i64, i64, i64, i64, i64, i32,
                                     i32, ctypes.POINTER(ptored_tuning), vp]
    lib.ptored_allreduce.restype = i32
    lib.ptored_ring_bounds.argtypes = [i64, i32, i32, ctypes.POINTER(i64)]
    lib.ptored_ring_bounds.restype = i32
    lib.ptored_reduce_scatter_ring.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i64,
                                               i32, i32, ctypes.POINTER(ptored_tuning), vp]
    lib.ptored_reduce_scatter_ring.restype = i32
    lib.ptored_accumulate_add.argtypes = [ctypes.POINTER(vp), i32, vp, i64, i64, i64, i64, i64,
                                          i32, ctypes.POINTER(ptored_tuning), vp]
    lib.ptored_accumulate_add.restype = i32
    lib.ptored_status_string.argtypes = [i32]
    lib.ptored_status_string.restype = ctypes.c_char_p
    lib.ptored_abi_version.restype = i32
    lib.ptored_max_ranks.restype = i32
    _lib = lib
    return lib


def pointer_array(ptrs: Sequence[int]) -> ctypes.Array:
    """A host array of device pointers in the ABI's form; the raw calls take
    one as is, so a caller that repeats a call can build it once."""
    return (ctypes.c_void_p * max(1, len(ptrs)))(*[int(p) for p in ptrs])


def _ptrs(srcs):
    return srcs if isinstance(srcs, ctypes.Array) else pointer_array(srcs)


def ptored_treduce(srcs: Sequence[int], nranks: int, root: int, dst: int, rows: int, cols: int,
                   ld: int, valid_rows: int, valid_cols: int, dtype: int, op: int,
                   stream: int) -> int:
    """Raw call: device pointers as ints; returns the status code."""
    return load().ptored_treduce(_ptrs(srcs), nranks, root, dst, rows, cols, ld, valid_rows,
                                 valid_cols, dtype, op, stream)


def ptored_treduce_ex(srcs: Sequence[int], nranks: int, root: int, dst: int, rows: int,
                      cols: int, ld: int, valid_rows: int, valid_cols: int, dtype: int, op: int,
                      tuning: Optional[ptored_tuning], stream: int) -> int:
    t = ctypes.byref(tuning) if tuning is not None else None
    return load().ptored_treduce_ex(_ptrs(srcs), nranks, root, dst, rows, cols, ld, valid_rows,
                                    valid_cols, dtype, op, t, stream)


def ptored_treduce_plan(srcs: Sequence[int], nranks: int, root: int, dst: int, rows: int,
                        cols: int, ld: int, valid_rows: int, valid_cols: int, dtype: int,
                        op: int, tuning: Optional[ptored_tuning] = None
                        ) -> Tuple[int, ptored_plan_info]:
    info = ptored_plan_info()
    t = ctypes.byref(tuning) if tuning is not None else None
    st = load().ptored_treduce_plan(_ptrs(srcs), nranks, root, dst, rows, cols, ld, valid_rows,
                                    valid_cols, dtype, op, t, ctypes.byref(info))
    return st, info


def ptored_allreduce(bufs: Sequence[int], nranks: int, root: int, rows: int, cols: int, ld: int,
                     valid_rows: int, valid_cols: int, dtype: int, op: int,
                     tuning: Optional[ptored_tuning], stream: int) -> int:
    t = ctypes.byref(tuning) if tuning is not None else None
    return load().ptored_allreduce(_ptrs(bufs), nranks, root, rows, cols, ld, valid_rows,
                                   valid_cols, dtype, op, t, stream)


def ptored_ring_bounds(count: int, nranks: int, dtype: int) -> Tuple[int, list]:
    out = (ctypes.c_int64 * (max(nranks, 0) + 1))()
    st = load().ptored_ring_bounds(count, nranks, dtype, out)
    return st, list(out)


def ptored_reduce_scatter_ring(srcs: Sequence[int], nranks: int, dsts: Sequence[int], count: int,
                               dtype: int, op: int, tuning: Optional[ptored_tuning],
                               stream: int) -> int:
    t = ctypes.byref(tuning) if tuning is not None else None
    return load().ptored_reduce_scatter_ring(_ptrs(srcs), nranks, _ptrs(dsts), count, dtype, op,
                                             t, stream)


def ptored_accumulate_add(srcs: Sequence[int], nranks: int, dst: int, rows: int, cols: int,
                          ld: int, valid_rows: int, valid_cols: int, dtype: int,
                          tuning: Optional[ptored_tuning], stream: int) -> int:
    t = ctypes.byref(tuning) if tuning is not None else None
    return load().ptored_accumulate_add(_ptrs(srcs), nranks, dst, rows, cols, ld, valid_rows,
                                        valid_cols, dtype, t, stream)


def ptored_status_string(status: int) -> str:
    return load().ptored_status_string(status).decode()


def ptored_abi_version() -> int:
    return load().ptored_abi_version()


def ptored_max_ranks() -> int:
    return load().ptored_max_ranks()


def tuning(flags: int = 0, blocks_per_cu: int = 0, max_launch_bytes: int = 0) -> ptored_tuning:
    return ptored_tuning(flags, blocks_per_cu, max_launch_bytes)


def _dtype_code(dtype) -> int:
    """C ABI code of a torch dtype or of one of "f32", "bf16", "f16", "i32"."""
    if isinstance(dtype, str):
        if dtype not in DTYPES:
            raise TypeError(f"unsupported dtype {dtype!r}; expected f32, bf16, f16 or i32")
        return DTYPES[dtype]
    import torch

    codes = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.int32: 3}
    if dtype not in codes:
        raise TypeError(f"unsupported dtype {dtype}; expected f32, bf16, f16 or i32")
    return codes[dtype]


def _torch_dtype_code(t) -> int:
    return _dtype_code(t.dtype)


def _op_code(op: str) -> int:
    if op not in OPS:
        raise ValueError(f"unsupported op {op!r}; expected sum, max, min or prod")
    return OPS[op]


def _geometry(t) -> Tuple[int, int, int]:
    if t.dim() == 1:
        return 1, t.shape[0], t.shape[0]
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("tensors must be 1-D or 2-D row-major with unit column stride")
    return t.shape[0], t.shape[1], t.stride(0)


def _check_group(tensors, ref, what: str):
    """Every tensor matches `ref` in dtype, geometry and device."""
    geo = _geometry(ref)
    for t in tensors:
        if t.dtype != ref.dtype or _geometry(t) != geo:
            raise ValueError(f"every {what} must match in dtype and geometry")
        if not t.is_cuda or t.device != ref.device:
            raise ValueError(f"every {what} must be on the same GPU")
    return geo


def _stream_handle(stream, device) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _raise_on(st: int) -> None:
    if st != PTORED_OK:
        raise PtoredError(st, ptored_status_string(st))


def treduce(srcs, dst, op: str = "sum", root: int = 0,
            valid: Optional[Tuple[int, int]] = None, tuning: Optional[ptored_tuning] = None,
            stream=None) -> None:
    """dst = fold of the source tensors over the valid rectangle, on the GPU.

    All tensors are on the current device with one dtype and one 2-D
    row-major geometry (``rows = size(0)``, ``cols = size(1)``,
    ``ld = stride(0)``).  ``valid`` defaults to the whole tensor.  The call is
    asynchronous on ``stream`` (default: torch's current stream).
    """
    import torch

    if len(srcs) == 0:
        raise ValueError("treduce needs at least one source")
    dt = _torch_dtype_code(dst)
    opc = _op_code(op)
    rows, cols, ld = _check_group(list(srcs) + [dst], dst, "tensor")
    vr, vc = (rows, cols) if valid is None else valid
    if vr == 0 or vc == 0:
        return  # an empty rectangle writes nothing (empty tensors have no storage)
    handle = _stream_handle(stream, dst.device)
    with torch.cuda.device(dst.device):
        _raise_on(ptored_treduce_ex([s.data_ptr() for s in srcs], len(srcs), root,
                                    dst.data_ptr(), rows, cols, ld, vr, vc, dt, opc, tuning,
                                    handle))


def allreduce(bufs, op: str = "sum", root: int = 0, valid: Optional[Tuple[int, int]] = None,
              tuning: Optional[ptored_tuning] = None, stream=None) -> None:
    """In place: every tensor's valid rectangle becomes the fold of all of them
    (root first, then ascending).  Geometry and stream as ``treduce``."""
    import torch

    if len(bufs) == 0:
        raise ValueError("allreduce needs at least one buffer")
    dt = _torch_dtype_code(bufs[0])
    opc = _op_code(op)
    rows, cols, ld = _check_group(bufs, bufs[0], "buffer")
    vr, vc = (rows, cols) if valid is None else valid
    if vr == 0 or vc == 0:
        return
    handle = _stream_handle(stream, bufs[0].device)
    with torch.cuda.device(bufs[0].device):
        _raise_on(ptored_allreduce([b.data_ptr() for b in bufs], len(bufs), root, rows, cols,
                                   ld, vr, vc, dt, opc, tuning, handle))


def ring_bounds(count: int, nranks: int, dtype) -> list:
    """The ring schedule's segment boundaries: nranks + 1 element offsets.
    ``dtype`` is a torch dtype or one of "f32", "bf16", "f16", "i32"."""
    st, out = ptored_ring_bounds(count, nranks, _dtype_code(dtype))
    _raise_on(st)
    return out


def reduce_scatter_ring(srcs, dsts, op: str = "sum", tuning: Optional[ptored_tuning] = None,
                        stream=None) -> None:
    """The ring reduce-scatter share on one GPU: the N contiguous source
    streams (all elements of each tensor) are cut into the ring's segments,
    and segment s, folded in ring order (ranks s+1, ..., s mod N), is written
    to dsts[s] at the same positions; nothing else of any dst is written."""
    import torch

    if len(srcs) == 0 or len(dsts) != len(srcs):
        raise ValueError("reduce_scatter_ring needs one dst per source")
    ref = srcs[0]
    for t in list(srcs) + list(dsts):
        if not t.is_contiguous():
            raise ValueError("reduce_scatter_ring streams must be contiguous")
        if t.dtype != ref.dtype or t.numel() != ref.numel():
            raise ValueError("every stream must match in dtype and length")
        if not t.is_cuda or t.device != ref.device:
            raise ValueError("every stream must be on the same GPU")
    dt = _torch_dtype_code(ref)
    opc = _op_code(op)
    if ref.numel() == 0:
        return
    handle = _stream_handle(stream, ref.device)
    with torch.cuda.device(ref.device):
        _raise_on(ptored_reduce_scatter_ring([s.data_ptr() for s in srcs], len(srcs),
                                             [d.data_ptr() for d in dsts], ref.numel(), dt,
                                             opc, tuning, handle))


def accumulate_add(srcs, dst, valid: Optional[Tuple[int, int]] = None,
                   tuning: Optional[ptored_tuning] = None, stream=None) -> None:
    """Push-with-add: dst += every source over the valid rectangle, by
    device-scope atomics, so pushes from other calls or streams into the same
    dst may land meanwhile.  The sources are folded in rank order first and
    the fold is added with one atomic per word; with
    ``tuning(flags=PTORED_ACC_PER_RANK)`` every source's elements are added
    with atomics of their own.  Geometry and stream as ``treduce``; dst may
    not be a source."""
    import torch

    if len(srcs) == 0:
        raise ValueError("accumulate_add needs at least one source")
    dt = _torch_dtype_code(dst)
    rows, cols, ld = _check_group(list(srcs) + [dst], dst, "tensor")
    vr, vc = (rows, cols) if valid is None else valid
    if vr == 0 or vc == 0:
        return
    handle = _stream_handle(stream, dst.device)
    with torch.cuda.device(dst.device):
        _raise_on(ptored_accumulate_add([s.data_ptr() for s in srcs], len(srcs), dst.data_ptr(),
                                        rows, cols, ld, vr, vc, dt, tuning, handle))
