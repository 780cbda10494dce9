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


def test_kernel_instances_are_matched_to_their_entry():
    w16 = W.find("n16_i32_4096x4096")
    w5 = W.find("n8_f16_8192x12288_valid8191x12287")
    cal = W.find("n1_i32_16384x16384_copy")
    k = "void ptored::treduce_kernel<{}>(ptored::KArgs)"
    assert bench.kernel_matches(k.format("3, 0, 4, 16, 1, 0, true, 0"), w16, "sum", "treduce")
    assert not bench.kernel_matches(k.format("3, 1, 4, 16, 1, 0, true, 0"), w16, "sum",
                                    "treduce")
    assert bench.kernel_matches(k.format("3, 1, 4, 16, 1, 0, true, 0"), w16, "max", "treduce")
    assert not bench.kernel_matches(k.format("3, 0, 4, 16, 1, 0, true, 1"), w16, "sum",
                                    "treduce")
    assert bench.kernel_matches(k.format("3, 0, 4, 16, 1, 0, true, 1"), w16, "sum",
                                "allreduce")
    assert bench.kernel_matches(k.format("3, 0, 4, 16, 1, 0, true, 2"), w16, "sum",
                                "accumulate_add")
    assert not bench.kernel_matches(k.format("3, 0, 4, 16, 1, 0, true, 2"), w16, "sum",
                                    "treduce")
    assert bench.kernel_matches(k.format("2, 1, 2, 8, 1, 1, true, 0"), w5, "max", "treduce")
    assert bench.kernel_matches(k.format("3, 0, 4, 1, 2, 0, true, 0"), cal, "sum", "treduce")
    assert not bench.kernel_matches(k.format("3, 0, 4, 1, 2, 0, true, 0"), w16, "sum",
                                    "treduce")
    assert bench.kernel_matches("void ptored::ring_kernel<3, 0, 4, 16>(ptored::RingArgs)", w16,
                                "sum", "reduce_scatter_ring")
    assert bench.kernel_matches("void ptored::accumulate_kernel<3, 4, 0, true>(ptored::KArgs)",
                                w16, "sum", "accumulate_add")
    assert not bench.kernel_matches("__amd_rocclr_copyBuffer", w16, "sum", "treduce")


def test_default_run_starts_with_the_headline_and_covers_every_config():
    pairs = bench.default_run()
    assert pairs[0] == (W.HEADLINE, "sum")
    want = {(w.name, op) for w in W.WORKLOADS.values() for op in w.ops}
    assert set(pairs) == want and len(pairs) == len(want)


def _write_csv(path, header, rows):
    import csv

    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_counters_scales_by_the_copy_in_the_same_run(monkeypatch, tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k16 = "void ptored::treduce_kernel<3, 0, 4, 16, 1, 0, true, 0>(ptored::KArgs)"
    kcopy = "void ptored::treduce_kernel<3, 0, 4, 1, 2, 0, true, 0>(ptored::KArgs)"
    gib_kib = 1 << 20
    _write_csv(tmp_path / "f" / "run_counter_collection.csv", hdr,
               [[k16, "FETCH_SIZE", 8 * 65536.0], [k16, "FETCH_SIZE", 8 * 65536.0],
                [kcopy, "FETCH_SIZE", gib_kib / 2], ["other", "FETCH_SIZE", 1.0]])
    _write_csv(tmp_path / "w" / "run_counter_collection.csv", hdr,
               [[k16, "WRITE_SIZE", 65536.0], [kcopy, "WRITE_SIZE", gib_kib]])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    out = tmp_path / "out.txt"
    monkeypatch.setattr(bench, "traffic_path", lambda wl, op, mode: str(out))

    class A:
        summarize_counters = (str(tmp_path / "f"), str(tmp_path / "w"))
        mode = "treduce"
        commands = ["cmd"]

    assert bench.summarize_counters(A) == 0
    vals = dict(ln.split(" = ") for ln in out.read_text().splitlines() if " = " in ln)
    assert float(vals["fetch_scale"]) == 2.0 and float(vals["write_scale"]) == 1.0
    # 16 x 64 MiB read (counted half, scaled by 2) + 64 MiB written
    assert int(vals["hbm_bytes_per_launch"]) == 17 * 64 * 2 ** 20
    assert vals["traffic_over_algorithmic"] == "1.0000"


def test_summarize_trace_pairs_each_entry_with_its_kernel(monkeypatch, tmp_path):
    import json

    hdr = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
           "StdDev"]
    k16 = "void ptored::treduce_kernel<3, 0, 4, 16, 1, 0, true, 0>(ptored::KArgs)"
    k16max = "void ptored::treduce_kernel<3, 1, 4, 16, 1, 0, true, 0>(ptored::KArgs)"
    _write_csv(tmp_path / "t" / "run_kernel_stats.csv", hdr,
               [[k16, 10, 1700000, 170000, 50, 160000, 180000, 1],
                [k16max, 10, 1720000, 172000, 50, 160000, 180000, 1]])
    line = {"metric": "m", "value": 6700.0, "ms_per_step": 0.171, "steps": 4, "warmup": 1,
            "config": {"workload": "n16_i32_4096x4096", "op": "sum", "mode": "treduce"},
            "configs": {"n16_i32_4096x4096:max": {
                "workload": "n16_i32_4096x4096", "op": "max", "ms_per_step": 0.1715,
                "gbs": 6650.0, "steps": 4, "warmup": 1}},
            "device": {"name": "gpu", "uuid": "u"}}
    log = tmp_path / "bench.log"
    log.write_text("noise\n" + json.dumps(line) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))

    class A:
        summarize_trace = str(tmp_path / "t")
        bench_log = str(log)
        commands = ["rocprofv3", "--kernel-trace"]

    assert bench.summarize_trace(A) == 0
    # the max entry's kernel (172 us) is longer than its step (171.5 us): flagged
    for op, avg, within in (("sum", "170.00", "true"), ("max", "172.00", "false")):
        text = (tmp_path / f"kernel_trace_n16_i32_4096x4096_{op}.txt").read_text()
        vals = dict(ln.split(" = ") for ln in text.splitlines() if " = " in ln)
        assert vals["kernel_average_us"] == avg
        assert vals["kernel_average_within_ms_per_step"] == within
        assert "uuid u" in text


def test_rotation_sends_every_step_to_hbm():
    """Input sets rotate only when one set fits in the Infinity Cache; the
    buffers a step writes rotate until 512 MiB are written between two uses
    of one, so a dst rewritten back to back cannot stay in the cache."""
    import bench
    from cross_rank_collective_amd import workloads as W
    head = W.find("n16_i32_4096x4096")
    assert bench.rotation(head, "treduce") == (1, 8, "hbm")            # 64 MiB dst
    assert bench.rotation(W.find("n8_bf16_8192x8192"), "treduce") == (1, 4, "hbm")
    assert bench.rotation(W.find("n8_f16_8192x12288_valid8191x12287"), "treduce") == (1, 3, "hbm")
    small = W.find("n4_f32_1024x1024_valid1000x1000")
    assert bench.rotation(small, "treduce") == (52, 128, "hbm")        # 20 MiB sets, 4 MiB dsts
    assert bench.rotation(head, "allreduce") == (1, 1, "hbm")          # writes all 16 buffers
    assert bench.rotation(head, "reduce_scatter_ring") == (8, 8, "hbm")  # writes 64 MiB per step
    assert bench.rotation(head, "accumulate_add") == (1, 8, "hbm")
    assert bench.rotation(head, "treduce", 1) == (1, 1, "cache-resident")
    assert bench.rotation(W.find("n2_f32_16x16"), "treduce")[2] == "cache-resident"
