"""Build libptored.so (HIP for gfx950) in-tree.

Every translation unit under csrc/ is compiled with hipcc in parallel and
linked into ``cross_rank_collective_amd/libptored.so``: the host code, one
unit per element type (copy and push-with-add kernels) and ``treduce_op.hip``
once per (element type, operator) pair (reduction and ring kernels).  Run as
``python -m cross_rank_collective_amd.build`` or through
``__graft_entry__.build()``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libptored.so")
BUILD_DIR = os.path.join(ROOT, "_build")

DTYPES = ("F32", "BF16", "F16", "I32")
OPS = ("SUM", "MAX", "MIN", "PROD")

# (source, object name, extra defines); the slowest units first.
UNITS = [("treduce_op.hip", f"treduce_op_{dt.lower()}_{op.lower()}",
          (f"-DPTORED_INST_DT=PTORED_{dt}", f"-DPTORED_INST_OP=PTORED_{op}"))
         for dt in ("BF16", "F16", "F32", "I32") for op in OPS]
UNITS += [(f"treduce_{dt.lower()}.hip", f"treduce_{dt.lower()}", ()) for dt in DTYPES]
UNITS += [("treduce_host.cpp", "treduce_host", ())]

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Keep the compiler from forming packed-FP32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _compile(unit) -> str:
    src, name, defines = unit
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc(), *CFLAGS, *defines, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name} ({src}):\n{res.stdout}\n{res.stderr}")
    return obj


def build(jobs: int = 0) -> str:
    """Compile every HIP unit for gfx950 and link libptored.so; returns its path.
    ``jobs`` = parallel compilers (0: one per CPU, at most 16)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    if jobs <= 0:
        jobs = min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, min(jobs, len(UNITS)))) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
