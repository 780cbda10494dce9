"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic
bytes of each mode, and the rule that stored HBM counter readings are quoted
only for the code they were taken on."""

import os
import subprocess
import sys

import bench
from cross_rank_collective_amd import workloads as W


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_algorithmic_bytes_of_each_mode():
    w = W.find("n16_i32_4096x4096")
    valid = 4096 * 4096 * 4
    assert bench.algorithmic_bytes(w, "treduce") == 17 * valid         # N reads + 1 write
    assert bench.algorithmic_bytes(w, "allreduce") == 32 * valid       # N reads + N writes
    assert bench.algorithmic_bytes(w, "reduce_scatter_ring") == 17 * valid
    assert bench.algorithmic_bytes(w, "accumulate_add") == 18 * valid  # + dst read and write
    assert bench.algorithmic_bytes(w, "memcpy") == 2 * valid
    # the ragged workload counts its valid rectangle only
    w5 = W.find("n8_f16_8192x12288_valid8191x12287")
    assert bench.algorithmic_bytes(w5, "treduce") == 9 * 8191 * 12287 * 2


def test_stored_traffic_only_for_the_code_it_was_taken_on(monkeypatch, tmp_path):
    path = tmp_path / "traffic_x_sum.txt"
    path.write_text("# a comment = ignored\nkernel_source_hash = abc\n"
                    "hbm_bytes_per_launch = 1234\n")
    monkeypatch.setattr(bench, "traffic_path", lambda wl, op, mode: str(path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.stored_traffic("x", "sum") == 1234
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abd")
    assert bench.stored_traffic("x", "sum") is None
    monkeypatch.setattr(bench, "traffic_path", lambda wl, op, mode: str(tmp_path / "none.txt"))
    assert bench.stored_traffic("x", "sum") is None


def test_comment_and_layout_edits_keep_the_source_hash():
    a = "int f(int x) { // add one\n  return x + 1; /* done */ }\n"
    b = "int f(int x) {\n    return x + 1;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("return x + 2;") != bench._code_only("return x + 1;")
    assert len(bench.kernel_source_hash()) == 16
