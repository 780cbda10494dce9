"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU (no GPU, no HIP runtime).

* The host code (argument checks, plans, launch splitting) is built with g++
  and linked with ``tests/sanitize/hip_stub.cpp``, which stands in for the
  HIP runtime and the kernel launches.  Two programs drive it through the C
  ABI: ``tests/c_abi_check.c`` (layouts, plans, ring bounds, error paths)
  and ``tests/sanitize/host_launches.c`` (every launch's byte windows checked
  against the buffers, over every kernel family, walk and the calls that
  split past 2 GiB).
* The oracle is built with the same sanitizers and its pins
  (``tests/test_oracle_pins.py``, ``tests/test_oracle_collectives.py``) run
  against that build in a child Python with the sanitizer runtimes
  preloaded.

Any sanitizer report ends the program with a nonzero status
(``-fno-sanitize-recover=all``, ``halt_on_error``).
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "cross_rank_collective_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(
    shutil.which("gcc") is None or shutil.which("g++") is None
    or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")),
    reason="needs gcc, g++ and the HIP headers")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def host_objects(tmp_path_factory):
    d = tmp_path_factory.mktemp("san_host")
    inc = ["-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}"]
    objs = []
    for src, name in ((os.path.join(CSRC, "treduce_host.cpp"), "host.o"),
                      (os.path.join(ROOT, "tests", "sanitize", "hip_stub.cpp"), "stub.o")):
        out = str(d / name)
        _run(["g++", "-std=c++17", "-Wall", "-Wextra", *SAN, *inc, "-c", src, "-o", out])
        objs.append(out)
    return d, inc, objs


@pytest.mark.parametrize("driver", ["sanitize/host_launches.c", "c_abi_check.c"])
def test_host_code_under_sanitizers(host_objects, driver):
    d, inc, objs = host_objects
    src = os.path.join(ROOT, "tests", driver)
    obj = str(d / (os.path.basename(driver) + ".o"))
    exe = str(d / os.path.basename(driver).replace(".c", ""))
    _run(["gcc", "-std=c11", "-Wall", "-Wextra", *SAN, *inc, "-c", src, "-o", obj])
    _run(["g++", *SAN, *objs, obj, "-o", exe])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120,
                         env={**os.environ, **ENV})
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr, res.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    import oracle

    lib = oracle.build(str(tmp_path / "libtreduce_oracle_san.so"), extra_flags=SAN)
    preload = ":".join(
        subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                       check=True).stdout.strip() for name in ("libasan.so", "libubsan.so"))
    env = {**os.environ, **ENV, "LD_PRELOAD": preload, "PTORED_ORACLE_LIB": lib}
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
           "not gpu", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_collectives.py")]
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert " passed" in res.stdout
