"""The library driven from a plain C program (tests/c_consumer_gpu.c): device
memory from hipMalloc, a HIP stream, the C ABI, and no torch in the process;
every call checked byte for byte against the oracle linked as a C library."""

import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _build(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    import oracle

    oracle._load()  # compiles the oracle if it is not built yet
    libdir = os.path.join(ROOT, "cross_rank_collective_amd")
    if not os.path.exists(os.path.join(libdir, "libptored.so")):
        pytest.fail("libptored.so is not built")
    odir = os.path.join(ROOT, "oracle")
    exe = str(tmp_path / "c_consumer_gpu")
    cmd = [gcc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
           os.path.join(HERE, "c_consumer_gpu.c"),
           "-L" + libdir, "-lptored", "-L" + odir, "-ltreduce_oracle",
           "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath," + libdir, "-Wl,-rpath," + odir, "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    subprocess.run(cmd, check=True)
    return exe


def test_c_program_against_the_oracle(tmp_path):
    exe = _build(tmp_path)
    print("running", exe, flush=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=150)
    sys.stdout.write(out.stdout[-2000:])
    assert out.returncode == 0 and "c consumer ok" in out.stdout, out.stdout[-3000:] + out.stderr
