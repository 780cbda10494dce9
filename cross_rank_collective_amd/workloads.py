"""Seeded synthetic inputs for the N-way reduction.

This module only draws input values.  It holds none of the reduction's
arithmetic and imports neither the GPU binding nor the CPU oracle, so both
sides can be fed identical inputs from it.

Every workload is a set of N equally shaped row-major buffers of
``rows x ld`` elements (``cols <= ld`` columns in use) with a valid rectangle
``valid_rows x valid_cols`` anchored at (0, 0).  Rank r of a workload draws
its whole buffer from ``numpy.random.default_rng(seed_base + r)`` (PCG64).

Value recipes (one per element type, chosen to resemble the shapes the
reduction meets in data-parallel training: uniform activations, small
Normal gradients, integer counters, and half-precision values with
saturated outliers):

* ``uniform_pm1``      f32   ``rng.random(float32) * 2 - 1``  (exactly in [-1, 1))
* ``normal_1e-2``      bf16  ``rng.standard_normal(float32) * 1e-2`` rounded to bf16
                             (round-to-nearest-even, via torch's CPU conversion)
* ``int_pm2^20``       i32   ``rng.integers(-2**20, 2**20, dtype=int32)``
* ``normal_sat``       f16   ``rng.standard_normal(float32)`` rounded to f16 (numpy RNE),
                             then every entry with ``rng.random() < 0.01`` becomes
                             +-65504 with a random sign (``rng.random() < 0.5`` -> minus)

Buffers are returned as numpy arrays of raw element bits: float32 for f32,
int32 for i32 and uint16 for bf16 / f16.
"""

from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

ESIZE = {"f32": 4, "bf16": 2, "f16": 2, "i32": 4}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "i32": np.int32}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    nranks: int
    dtype: str
    ops: Tuple[str, ...]
    rows: int
    cols: int
    ld: int
    valid_rows: int
    valid_cols: int
    root: int
    recipe: str
    seed_base: int

    @property
    def esize(self) -> int:
        return ESIZE[self.dtype]

    @property
    def buffer_elems(self) -> int:
        return self.rows * self.ld

    @property
    def valid_bytes(self) -> int:
        return self.valid_rows * self.valid_cols * self.esize

    @property
    def algorithmic_bytes(self) -> int:
        """N reads of every valid element plus one write of it."""
        return (self.nranks + 1) * self.valid_bytes


# The five workloads: tiny tile, cache-sized f32 with a sub-rectangle,
# gradient-sized bf16, 16-rank i32, and ragged f16 with saturated entries.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("n2_f32_16x16", 2, "f32", ("sum",), 16, 16, 16, 16, 16, 0,
                 "uniform_pm1", 1000),
        Workload("n4_f32_1024x1024_valid1000x1000", 4, "f32", ("sum", "max", "min"),
                 1024, 1024, 1024, 1000, 1000, 0, "uniform_pm1", 2000),
        Workload("n8_bf16_8192x8192", 8, "bf16", ("sum",), 8192, 8192, 8192, 8192, 8192, 0,
                 "normal_1e-2", 3000),
        Workload("n16_i32_4096x4096", 16, "i32", ("sum", "max"), 4096, 4096, 4096, 4096, 4096,
                 0, "int_pm2^20", 4000),
        Workload("n8_f16_8192x12288_valid8191x12287", 8, "f16", ("max",), 8192, 12288, 12288,
                 8191, 12287, 0, "normal_sat", 5000),
    ]
}

# The largest N-way reduce: 16 ranks.
HEADLINE = "n16_i32_4096x4096"

# A plain 1 GiB copy (one rank): reads and writes a known number of bytes,
# used to scale hardware traffic counters to bytes.
CALIBRATION = {
    w.name: w
    for w in [
        Workload("n1_i32_16384x16384_copy", 1, "i32", ("sum",), 16384, 16384, 16384, 16384,
                 16384, 0, "int_pm2^20", 6000),
    ]
}


def find(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    if name in CALIBRATION:
        return CALIBRATION[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS) + sorted(CALIBRATION)}")


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch  # CPU conversion only; rounds to nearest, ties to even

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(recipe: str, n: int, seed: int) -> np.ndarray:
    """n values of one recipe from PCG64(seed), as raw element bits."""
    rng = np.random.default_rng(seed)
    if recipe == "uniform_pm1":
        return rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if recipe == "normal_1e-2":
        return _f32_to_bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(1e-2))
    if recipe == "int_pm2^20":
        return rng.integers(-(2 ** 20), 2 ** 20, size=n, dtype=np.int32)
    if recipe == "normal_sat":
        v = rng.standard_normal(n, dtype=np.float32).astype(np.float16)
        hit = rng.random(n, dtype=np.float32) < np.float32(0.01)
        neg = rng.random(n, dtype=np.float32) < np.float32(0.5)
        v[hit] = np.where(neg[hit], np.float16(-65504.0), np.float16(65504.0))
        return v.view(np.uint16)
    raise ValueError(f"unknown recipe {recipe!r}")


def draw_device(recipe: str, n: int, seed: int, device: str = "cuda"):
    """n values of one recipe drawn on the device with torch's generator
    seeded by `seed` (for buffers too large to draw on the host), as a tensor
    of raw element bits: int32 for the 4-byte types, int16 for the 2-byte
    ones.  Same distributions as ``draw``; not the same values."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    if recipe == "uniform_pm1":
        return (torch.rand(n, generator=g, device=device) * 2.0 - 1.0).view(torch.int32)
    if recipe == "normal_1e-2":
        x = torch.randn(n, generator=g, device=device) * 1e-2
        return x.to(torch.bfloat16).view(torch.int16)
    if recipe == "int_pm2^20":
        return torch.randint(-(2 ** 20), 2 ** 20, (n,), generator=g, device=device,
                             dtype=torch.int32)
    if recipe == "normal_sat":
        v = torch.randn(n, generator=g, device=device).to(torch.float16)
        hit = torch.rand(n, generator=g, device=device) < 0.01
        neg = torch.rand(n, generator=g, device=device) < 0.5
        sat = torch.where(neg, -65504.0, 65504.0).to(torch.float16)
        return torch.where(hit, sat, v).view(torch.int16)
    raise ValueError(f"unknown recipe {recipe!r}")


def make_sources(w: Workload, threads: int = 8) -> List[np.ndarray]:
    """The N rank buffers of a workload, each ``rows x ld`` elements.

    Ranks are drawn on a small thread pool (numpy's generators release the
    GIL while filling); each rank has its own generator, so the result does
    not depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor

    with ThreadPoolExecutor(max(1, min(threads, w.nranks))) as ex:
        return list(ex.map(lambda r: draw(w.recipe, w.buffer_elems, w.seed_base + r),
                           range(w.nranks)))


def sentinel_bits(dtype: str) -> int:
    """All-ones bit pattern: -1 for i32, a NaN pattern for the float types."""
    return -1 if dtype in ("f32", "i32") else 0xFFFF


def sentinel_buffer(dtype: str, n: int) -> np.ndarray:
    if dtype == "f32":
        return np.full(n, -1, dtype=np.int32).view(np.float32)
    if dtype == "i32":
        return np.full(n, -1, dtype=np.int32)
    return np.full(n, 0xFFFF, dtype=np.uint16)
