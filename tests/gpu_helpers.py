"""Helpers for the GPU parity tests: device buffers with guard bands, the
oracle call on the same inputs, and bitwise comparison (NaN by NaN-ness)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from cross_rank_collective_amd import binding as B
from cross_rank_collective_amd import workloads as W

GUARD = 4096  # bytes of sentinel before and after every dst view
STORAGE = W.STORAGE
ESIZE = W.ESIZE


def say(*args):
    print("[case]", *args, file=sys.stderr, flush=True)


class DevBuf:
    """A device byte buffer holding one element array at a chosen byte offset
    (for misaligned pointers), surrounded by guard bands of one fill byte."""

    def __init__(self, nbytes: int, offset: int = 0, fill: int = 0xFF):
        assert 0 <= offset < 2048
        self.nbytes = nbytes
        self.start = GUARD + offset
        self.t = torch.full((GUARD + offset + nbytes + GUARD,), fill, dtype=torch.uint8,
                            device="cuda")
        self.fill = fill

    @property
    def ptr(self) -> int:
        return self.t.data_ptr() + self.start

    def upload(self, arr: np.ndarray):
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == self.nbytes, (raw.size, self.nbytes)
        self.t[self.start:self.start + self.nbytes].copy_(torch.from_numpy(raw.copy()))

    def download_all(self) -> np.ndarray:
        return self.t.cpu().numpy()

    def download(self, dtype: str) -> np.ndarray:
        full = self.download_all()
        return full[self.start:self.start + self.nbytes].view(STORAGE[dtype])

    def guards_intact(self) -> bool:
        full = self.download_all()
        return bool(np.all(full[:self.start] == self.fill)
                    and np.all(full[self.start + self.nbytes:] == self.fill))


def bits(dtype: str, a: np.ndarray) -> np.ndarray:
    if dtype in ("f32", "i32"):
        return a.view(np.uint32).astype(np.uint64)
    return a.view(np.uint16).astype(np.uint64)


def isnan_bits(dtype: str, b: np.ndarray) -> np.ndarray:
    if dtype == "i32":
        return np.zeros(b.shape, dtype=bool)
    if dtype == "f32":
        return ((b >> 23) & 0xFF == 0xFF) & (b & 0x7FFFFF != 0)
    if dtype == "f16":
        return ((b >> 10) & 0x1F == 0x1F) & (b & 0x3FF != 0)
    return ((b >> 7) & 0xFF == 0xFF) & (b & 0x7F != 0)


def compare(dtype: str, got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Mask of element positions that agree (bits equal; NaN matches NaN)."""
    g, w = bits(dtype, got), bits(dtype, want)
    ng, nw = isnan_bits(dtype, g), isnan_bits(dtype, w)
    return np.where(ng | nw, ng & nw, g == w)


def valid_mask(rows: int, ld: int, vr: int, vc: int, size: int) -> np.ndarray:
    m = np.zeros(rows * ld, dtype=bool)
    m.reshape(rows, ld)[:vr, :vc] = True
    return m[:size]


def run_gpu(srcs, dtype: str, op: str, root: int, rows: int, cols: int, ld: int, vr: int,
            vc: int, *, offsets=None, dst_offset: int = 0, tuning=None, alias: int = -1,
            label: str = ""):
    """Upload sources, run ptored_treduce_ex, return (dst DevBuf, status)."""
    es = ESIZE[dtype]
    size = (rows - 1) * ld + cols if rows > 0 else 0
    nbytes = max(size, 1) * es
    n = len(srcs)
    offsets = offsets or [0] * n
    bufs = []
    for s, off in zip(srcs, offsets):
        assert s.size >= size
        b = DevBuf(nbytes, off, fill=0xA5)
        b.upload(s[:max(size, 1)])
        bufs.append(b)
    if alias >= 0:
        dst = bufs[alias]
    else:
        dst = DevBuf(nbytes, dst_offset, fill=0xFF)
    say(label, f"dtype={dtype} op={op} N={n} root={root} rows={rows} cols={cols} ld={ld} "
               f"valid={vr}x{vc} offs={offsets[:4]} dst_off={dst_offset} alias={alias} "
               f"flags={getattr(tuning, 'flags', 0)}")
    st = B.ptored_treduce_ex([b.ptr for b in bufs], n, root, dst.ptr, rows, cols, ld, vr, vc,
                             B.DTYPES[dtype], B.OPS[op], tuning,
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return dst, st, bufs


def oracle_reduce(srcs, dtype, op, root, rows, cols, ld, vr, vc, fill_dst):
    size = (rows - 1) * ld + cols if rows > 0 else 0
    d = fill_dst(max(size, 1))
    oracle.treduce([np.ascontiguousarray(s[:max(size, 1)]) for s in srcs], d, root=root,
                   dtype=dtype, op=op, rows=rows, cols=cols, ld=ld, valid_rows=vr,
                   valid_cols=vc)
    return d


def host_threads() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of a box)."""
    import os

    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_reduce_banded(srcs, dtype, op, root, rows, cols, ld, vr, vc):
    """The oracle over a whole (large) workload into a sentinel-filled buffer,
    in row bands on the host cores."""
    size = (rows - 1) * ld + cols if rows > 0 else 0
    d = sentinel(dtype, max(size, 1))
    oracle.treduce_banded([np.ascontiguousarray(s[:max(size, 1)]) for s in srcs], d, root=root,
                          dtype=dtype, op=op, rows=rows, cols=cols, ld=ld, valid_rows=vr,
                          valid_cols=vc, threads=host_threads())
    return d


def sentinel(dtype: str, n: int) -> np.ndarray:
    return np.full(n * ESIZE[dtype], 0xFF, dtype=np.uint8).view(STORAGE[dtype])
