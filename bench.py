"""Benchmark of the N-way reduction on one MI355X.

One step = one ptored_treduce call over the whole workload (every source
read once, dst written once), inputs resident in HBM and every step's output
written to HBM (dst rotated over enough buffers that none is still in the
256 MB Infinity Cache when it is written again).  Prints ONE JSON line:
effective HBM GB/s = (N+1) * valid bytes / time of the 16-rank i32 Sum
workload (the largest N-way reduce), with the roofline of its kernel and the
CPU oracle timed on a bounded sample as a baseline, and beside it:

* ``configs``: every other workload and operator, timed the same way in the
  same process, each with its fraction of the HBM peak and ``gpu_bit_exact``:
  whether every valid element of its output equals the oracle's (and every
  other element kept its sentinel).  Steps whose launch moves less than
  64 MiB are timed over at least 1000 steps, and the 1000 x 1000 workload,
  which fits the 256 MB Infinity Cache, rotates over copies of its buffers
  so that every step reads from HBM;
* ``ceilings``: the runtime's device-to-device hipMemcpyAsync of 1 GiB and
  the library's own copy kernel (one source) over 1 GiB, in the same run;
* ``device``: the GPU the figures come from.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op OP]
                    [--mode treduce|allreduce|reduce_scatter_ring|accumulate_add|memcpy]
                    [--sets S] [--headline-only] [--no-cpu-baseline]
    python bench.py --summarize-trace DIR --bench-log LOG --commands CMD
    python bench.py --summarize-counters FETCH_DIR WRITE_DIR [--mode M] --commands CMD...

The default mode is the reduction itself (dst = fold of the N sources); the
other modes time the collective variants on the named workload: the in-place
allreduce (N reads + N writes per valid element), the ring reduce-scatter
share over the whole buffer as one stream (N reads + 1 write per element)
and push-with-add by atomics (N source reads + one read and one write of dst
per element, the least any order of the additions must move); memcpy times
the runtime's device-to-device copy of one buffer.

Steps default to 200 timed calls after W warm-up calls, and to 1000 for a
workload whose step moves less than 64 MiB (the two small ones), whose
launches last a few microseconds.

The summarizers turn rocprofv3 output of a bench command into the files
under profiles/: --summarize-trace one kernel-trace summary per entry of the
bench line (with that run's bench figures and device), --summarize-counters
one HBM-traffic summary per entry from a FETCH_SIZE run and a WRITE_SIZE run
(scaled by the counters of the 1 GiB copy the same runs launch).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
PROFILES = os.path.join(ROOT, "profiles")
MODES = ["treduce", "allreduce", "reduce_scatter_ring", "accumulate_add", "memcpy"]
MALL_BYTES = 256 << 20   # MI355X Infinity Cache
ROTATE_BYTES = 1 << 30   # rotate input sets until the steps touch at least this much
# Rotate the buffers a step writes until this many bytes are written between
# two uses of one of them: a dst rewritten back to back stays in the Infinity
# Cache and never reaches HBM, which a real loop (other work between two
# reductions) does not see.
WRITE_ROTATE_BYTES = 2 * MALL_BYTES
MAX_DSTS = 256
SMALL_STEP_BYTES = 64 << 20  # steps moving less than this are timed 1000 times by default
MAX_SETS = 64
# The kernel each mode launches (one launch per call at the bench's sizes).
MODE_KERNEL = {"treduce": "treduce_kernel", "allreduce": "treduce_kernel",
               "reduce_scatter_ring": "ring_kernel", "accumulate_add": "treduce_kernel",
               "memcpy": "copyBuffer"}


# The metric of each mode: the reduction's is the headline metric; the others
# name their own algorithmic bytes.
METRIC = {
    "treduce": "effective HBM GB/s ((N+1)\u00b7valid bytes / time) and % of MI355X peak",
    "allreduce": "effective HBM GB/s (2N\u00b7valid bytes / time) and % of MI355X peak",
    "reduce_scatter_ring": "effective HBM GB/s ((N+1)\u00b7stream bytes / time) and % of MI355X peak",
    "accumulate_add": "effective HBM GB/s ((N+2)\u00b7valid bytes / time) and % of MI355X peak",
    "memcpy": "device-to-device copy GB/s (2\u00b7buffer bytes / time) and % of MI355X peak",
}


def algorithmic_bytes(w, mode: str) -> int:
    """Bytes a call must move: N reads + 1 write of every valid element
    (reduce); N reads + N writes (in-place allreduce); N reads + 1 write of
    every element of the stream (ring reduce-scatter); N reads + one read and
    one write of dst (push-with-add)."""
    if mode == "treduce":
        return w.algorithmic_bytes
    if mode == "allreduce":
        return 2 * w.nranks * w.valid_bytes
    if mode == "reduce_scatter_ring":
        return (w.nranks + 1) * w.buffer_elems * w.esize
    if mode == "memcpy":  # context: the runtime's copy of one source buffer into dst
        return 2 * w.buffer_elems * w.esize
    return (w.nranks + 2) * w.valid_bytes


def traffic_path(workload: str, op: str, mode: str) -> str:
    suffix = "" if mode == "treduce" else f"_{mode}"
    return os.path.join(PROFILES, f"traffic_{workload}_{op}{suffix}.txt")


CSRC = os.path.join(ROOT, "cross_rank_collective_amd", "csrc")


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (the code
    in these files has no string literal holding comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the library's code (comments and layout ignored); the stored
    HBM counter readings are only quoted while the code is the one they
    were taken on."""
    h = hashlib.sha256()
    for fn in sorted(os.listdir(CSRC)):
        if fn.endswith((".hpp", ".hip", ".h", ".cpp")):
            h.update(fn.encode())
            h.update(_code_only(open(os.path.join(CSRC, fn), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, op: str, mode: str = "treduce"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none for this kernel source."""
    path = traffic_path(workload, op, mode)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


DT_CODE = {"f32": 0, "bf16": 1, "f16": 2, "i32": 3}
OP_CODE = {"sum": 0, "max": 1, "min": 2, "prod": 3}


def kernel_template(name: str):
    """(kernel, [template arguments]) of a demangled kernel name such as
    ``void ptored::treduce_kernel<3, 0, 4, 16, 1, 0, true, false>(ptored::KArgs)``,
    or None for a name without template arguments."""
    m = re.search(r"(\w+)<([^<>]*)>\(", name)
    if not m:
        return None
    return m.group(1), [a.strip() for a in m.group(2).split(",")]


# The store-mode argument of treduce_kernel: into dst, into every source
# (the in-place allreduce), added into dst (push-with-add).
STORE_MODE = {"treduce": "0", "allreduce": "1", "accumulate_add": "2"}


def kernel_matches(name: str, w, op: str, mode: str) -> bool:
    """Whether a kernel instance is the one a call of `mode` on workload `w`
    with operator `op` launches: the reduction, the allreduce and the default
    push-with-add run treduce_kernel<type, op, esize, N, ..., store mode>
    (N = 0 for the runtime rank loop above 16; N = 1 is the copy; push-with-
    add is a Sum), the ring ring_kernel<type, op, esize, N>, per-rank push-
    with-add accumulate_kernel<type, esize, ...>, memcpy the runtime's copy
    kernel."""
    if mode == "memcpy":
        return "copyBuffer" in name
    t = kernel_template(name)
    if t is None:
        return False
    kern, args = t
    dt, es = str(DT_CODE[w.dtype]), str(w.esize)
    nr = str(w.nranks if w.nranks <= 16 else 0)
    if mode == "reduce_scatter_ring":
        return kern == "ring_kernel" and args == [dt, str(OP_CODE[op]), es, nr]
    if mode == "accumulate_add" and kern == "accumulate_kernel":
        return args[:2] == [dt, es]
    opc = str(OP_CODE["sum" if mode == "accumulate_add" else op])
    return (kern == "treduce_kernel" and args[:4] == [dt, opc, es, nr]
            and args[-1] == STORE_MODE[mode])


def default_run():
    """(workload, op) pairs the default run times: the headline first, then
    every other workload and operator."""
    from cross_rank_collective_amd import workloads as W

    head = W.WORKLOADS[W.HEADLINE]
    pairs = [(head.name, op) for op in head.ops]
    for w in W.WORKLOADS.values():
        pairs += [(w.name, op) for op in w.ops if (w.name, op) not in pairs]
    return pairs


def _csv_rows(directory: str, suffix: str):
    import csv
    import glob

    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(path) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _counter_means_kib(directory: str, counter: str):
    """{kernel name: mean per-dispatch value of `counter`} from a rocprofv3
    --pmc run written with -f csv under `directory`."""
    acc = {}
    for row in _csv_rows(directory, "counter_collection.csv"):
        if row.get("Counter_Name") == counter:
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _mean_for(means, w, op, mode):
    vals = [v for k, v in means.items() if kernel_matches(k, w, op, mode)]
    if len(vals) != 1:
        return None
    return vals[0]


def summarize_counters(args) -> int:
    """Write the HBM-traffic summary of every (workload, op) whose kernel
    appears in two rocprofv3 --pmc runs of one bench command (FETCH_SIZE,
    then WRITE_SIZE), each counter scaled by what it reads for the library's
    1 GiB copy, which every bench run also launches (the copy ceiling)."""
    from cross_rank_collective_amd import workloads as W

    fetch_dir, write_dir = args.summarize_counters
    fetch_m = _counter_means_kib(fetch_dir, "FETCH_SIZE")
    write_m = _counter_means_kib(write_dir, "WRITE_SIZE")
    cal = W.CALIBRATION["n1_i32_16384x16384_copy"]
    cal_fetch = _mean_for(fetch_m, cal, "sum", "treduce")
    cal_write = _mean_for(write_m, cal, "sum", "treduce")
    if cal_fetch is None or cal_write is None:
        raise RuntimeError("the 1 GiB copy kernel is missing from the counter runs")
    copy_bytes = cal.valid_bytes
    fetch_scale = copy_bytes / (cal_fetch * 1024.0)
    write_scale = copy_bytes / (cal_write * 1024.0)
    mode = args.mode
    if mode == "treduce":
        pairs = default_run()
    elif mode == "accumulate_add":  # a Sum whatever the workload's operators
        pairs = [(w.name, "sum") for w in W.WORKLOADS.values()]
    else:
        pairs = [(w.name, op) for w in W.WORKLOADS.values() for op in w.ops]
    written = 0
    for wl, op in pairs:
        w = W.find(wl)
        fetch = _mean_for(fetch_m, w, op, mode)
        write = _mean_for(write_m, w, op, mode)
        if fetch is None or write is None:
            continue
        kernel = MODE_KERNEL[mode]
        algo = algorithmic_bytes(w, mode)
        traffic = fetch * 1024.0 * fetch_scale + write * 1024.0 * write_scale
        lines = [
            f"# HBM traffic per launch of {kernel}, workload {w.name}, op {op}, mode {mode}",
            "# from rocprofv3 counters (KiB per dispatch, mean over the run's dispatches of",
            "# this kernel instance), scaled by the same counters read on the library's",
            f"# 1 GiB copy in the same runs ({cal.name}: {copy_bytes} bytes read and written).",
            "# commands (each its own run, from the repository root):",
        ]
        lines += [f"#   {c}" for c in args.commands]
        lines += [
            f"kernel_source_hash = {kernel_source_hash()}",
            f"fetch_kib_per_dispatch = {fetch:.1f}",
            f"write_kib_per_dispatch = {write:.1f}",
            f"copy_fetch_kib_per_dispatch = {cal_fetch:.1f}",
            f"copy_write_kib_per_dispatch = {cal_write:.1f}",
            f"fetch_scale = {fetch_scale:.5f}",
            f"write_scale = {write_scale:.5f}",
            f"hbm_bytes_per_launch = {traffic:.0f}",
            f"algorithmic_bytes_per_launch = {algo}",
            f"traffic_over_algorithmic = {traffic / algo:.4f}",
        ]
        text = "\n".join(lines) + "\n"
        with open(traffic_path(w.name, op, mode), "w") as fh:
            fh.write(text)
        print(text, end="")
        written += 1
    if written == 0:
        raise RuntimeError("no kernel of a known workload in the counter runs")
    return 0


def _bench_line(path: str):
    line = None
    for text in open(path):
        text = text.strip()
        if text.startswith("{") and '"metric"' in text:
            line = json.loads(text)
    if line is None:
        raise RuntimeError(f"no bench line in {path}")
    return line


def summarize_trace(args) -> int:
    """Write one kernel-trace summary per (workload, op) of a bench run
    profiled with rocprofv3 --kernel-trace --stats: the kernel instance's
    call count and durations, the bandwidth from its average duration, the
    same run's bench figures for that entry, and the device they come from."""
    from cross_rank_collective_amd import workloads as W

    stats = _csv_rows(args.summarize_trace, "kernel_stats.csv")
    agents = [a for a in _csv_rows(args.summarize_trace, "agent_info.csv")
              if a.get("Agent_Type") == "GPU"]
    line = _bench_line(args.bench_log)
    mode = line["config"]["mode"]
    entries = [dict(line["config"], ms_per_step=line["ms_per_step"], gbs=line["value"],
                    steps=line["steps"], warmup=line["warmup"])]
    entries += [dict(c, workload=c["workload"], op=c["op"]) for c in
                line.get("configs", {}).values()]
    dev = line.get("device", {})
    agent = agents[0] if agents else {}
    written = 0
    for e in entries:
        w = W.find(e["workload"])
        op = e["op"]
        rows = [r for r in stats if kernel_matches(r["Name"], w, op, mode)]
        if not rows:
            continue
        calls = sum(int(r["Calls"]) for r in rows)
        avg_ns = sum(float(r["TotalDurationNs"]) for r in rows) / calls
        algo = algorithmic_bytes(w, mode)
        gbs = algo / (avg_ns * 1e-9) / 1e9
        suffix = "" if mode == "treduce" else f"_{mode}"
        out = os.path.join(PROFILES, f"kernel_trace_{w.name}_{op}{suffix}.txt")
        text = [
            f"# rocprofv3 kernel-trace statistics, workload {w.name}, op {op}, mode {mode}",
            f"# command (from the repository root): {' '.join(args.commands)}",
            f"# bench entry: {e['steps']} timed steps after {e['warmup']} warm-up steps, then as "
            "many timed one by one; one launch per step",
            f"# device: {dev.get('name', '?')} {dev.get('arch', '?')} uuid {dev.get('uuid', '?')} "
            f"pci {dev.get('pci', '?')} host {dev.get('host', '?')}; profiler agent gpu_id "
            f"{agent.get('Gpu_Id', '?')} location {agent.get('Location_Id', '?')}",
            "# name | calls | average ns | min ns | max ns | stddev ns",
        ]
        for r in rows:
            text.append(f"{r['Name']} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                        f"{r['MinNs']} | {r['MaxNs']} | {float(r['StdDev']):.0f}")
        text += [
            f"kernel_source_hash = {kernel_source_hash()}",
            f"algorithmic_bytes_per_launch = {algo}",
            f"kernel_average_us = {avg_ns / 1e3:.2f}",
            f"kernel_gbs_from_trace = {gbs:.1f}",
            f"kernel_frac_from_trace = {gbs / HBM_PEAK_GBS:.4f}",
            f"bench_ms_per_step_same_run = {e['ms_per_step']}",
            f"bench_gbs_same_run = {e['gbs']}",
            f"kernel_average_within_ms_per_step = "
            f"{str(avg_ns / 1e6 <= e['ms_per_step']).lower()}",
        ]
        with open(out, "w") as fh:
            fh.write("\n".join(text) + "\n")
        print(f"wrote {out}: {avg_ns / 1e3:.2f} us, {gbs:.1f} GB/s, bench {e['gbs']} GB/s")
        written += 1
    if written == 0:
        raise RuntimeError("no kernel of the bench run in the trace")
    return 0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_threads() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of a box)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, op, srcs, gpu_dst_bits, target_s: float = 10.0):
    """Time the oracle as written on the first rows of the same workload:
    on one thread, sized to about `target_s` seconds, and on every host core
    (row bands, one oracle call per band and thread) for about as long; check
    the GPU rows against it bit for bit."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from cross_rank_collective_amd import workloads as W

    def band(rows, r0, r1, dst):
        # rows [r0, r1) of the first `rows` rows, into dst (ctypes drops the GIL)
        off = r0 * w.ld
        size = (r1 - r0 - 1) * w.ld + w.cols
        sub = [s[off:off + size] for s in srcs]
        oracle.treduce(sub, dst[off:off + size], root=w.root, dtype=w.dtype, op=op,
                       rows=r1 - r0, cols=w.cols, ld=w.ld, valid_rows=r1 - r0,
                       valid_cols=w.valid_cols)

    def run(rows, threads=1, pool=None):
        size = (rows - 1) * w.ld + w.cols
        dst = W.sentinel_buffer(w.dtype, size)
        t0 = time.perf_counter()
        if threads == 1:
            band(rows, 0, rows, dst)
        else:
            cuts = [rows * k // threads for k in range(threads + 1)]
            list(pool.map(lambda k: band(rows, cuts[k], cuts[k + 1], dst),
                          [k for k in range(threads) if cuts[k + 1] > cuts[k]]))
        return time.perf_counter() - t0, dst

    def timed(rows, threads, pool, budget):
        t = run(rows, threads, pool)[0]
        repeats = 1
        if t < budget / 2:
            repeats = int(min(400, budget // max(t, 1e-6)))
            total = t
            for _ in range(repeats - 1):
                total += run(rows, threads, pool)[0]
            t = total / repeats
        return t, repeats

    probe_rows = min(w.valid_rows, 8)
    t_probe, _ = run(probe_rows)
    rows = int(min(w.valid_rows, max(probe_rows, probe_rows * target_s / max(t_probe, 1e-6))))
    t1, dst = run(rows)
    # When the whole workload takes well under the target, repeat it and
    # report the mean, so the baseline is not a single short timing.
    repeats1 = 1
    if rows == w.valid_rows and t1 < target_s / 2:
        t1, repeats1 = timed(rows, 1, None, target_s)
    threads = host_threads()
    with ThreadPoolExecutor(threads) as pool:
        tn, repeats_n = timed(rows, threads, pool, target_s)
        _, dst_n = run(rows, threads, pool)
    nbytes = (w.nranks + 1) * rows * w.valid_cols * w.esize
    m = np.zeros((rows, w.ld), dtype=bool)
    m[:, :w.valid_cols] = True
    m = m.reshape(-1)[:dst.size]
    gpu = gpu_dst_bits[:dst.size]
    same = np.array_equal(gpu.view(np.uint8).reshape(dst.size, -1)[m],
                          dst.view(np.uint8).reshape(dst.size, -1)[m])
    bands_same = np.array_equal(dst.view(np.uint8), dst_n.view(np.uint8))
    return {
        "value": round(nbytes / tn / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"first {rows} of {w.valid_rows} valid rows ({rows * w.valid_cols} elements x "
                  f"{w.nranks} ranks), split in {threads} row bands over {threads} threads, "
                  f"mean of {repeats_n} run(s) of {tn:.4f} s; one thread: mean of {repeats1} "
                  f"run(s) of {t1:.3f} s; {cpu_model()}",
        "value_1_thread": round(nbytes / t1 / 1e9, 4),
        "seconds": round(tn, 4),
        "gpu_rows_bit_exact": bool(same and bands_same),
    }


def oracle_full_check(w, op, srcs, gpu_bits) -> bool:
    """Whether every valid element of the GPU's output equals the oracle's
    (computed over the whole workload in row bands on the host cores) and
    every element outside the valid rectangle kept its sentinel.  Part of
    the CPU leg: runs after the GPU timing of the entry, on host copies."""
    import oracle
    from cross_rank_collective_amd import workloads as W

    want = W.sentinel_buffer(w.dtype, w.buffer_elems)
    oracle.treduce_banded(srcs, want, root=w.root, dtype=w.dtype, op=op, rows=w.rows,
                          cols=w.cols, ld=w.ld, valid_rows=w.valid_rows,
                          valid_cols=w.valid_cols, threads=host_threads())
    return bool(np.array_equal(gpu_bits.view(np.uint8), want.view(np.uint8)))


def time_steps(torch, stream, step, steps: int, warmup: int):
    """Mean milliseconds per step over `steps` back-to-back steps after
    `warmup` untimed ones (HIP events on the launch stream), and the sorted
    per-step times of a second pass with an event pair around every step."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / steps
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    for a_ev, b_ev in marks:
        a_ev.record(stream)
        step()
        b_ev.record(stream)
    torch.cuda.synchronize()
    return ms_step, sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in marks)


def rotation(w, mode: str, sets_arg: int = 0):
    """(input sets, dsts, residency) the steps of one entry rotate over.
    Automatic (sets_arg <= 0): input sets when one set fits in the Infinity
    Cache, until the steps touch ROTATE_BYTES; the buffers a step writes --
    dst, or the sources themselves in the in-place modes -- until
    WRITE_ROTATE_BYTES are written between two uses of one.  sets_arg > 0:
    exactly that many of each.  residency is "hbm" when every step reads
    from and writes to HBM."""
    buf_bytes = w.buffer_elems * w.esize
    set_bytes = (2 if mode == "memcpy" else w.nranks + 1) * buf_bytes
    in_place = mode in ("allreduce", "reduce_scatter_ring")
    written = w.nranks * buf_bytes if mode == "allreduce" else buf_bytes
    nsets, ndst = sets_arg, sets_arg
    if sets_arg <= 0:
        nsets = 1 if set_bytes >= MALL_BYTES else min(MAX_SETS, -(-ROTATE_BYTES // set_bytes))
        if in_place:
            nsets = max(nsets, -(-WRITE_ROTATE_BYTES // written))
        ndst = nsets if in_place else max(nsets, min(MAX_DSTS, -(-WRITE_ROTATE_BYTES // written)))
    reads_hbm = set_bytes >= MALL_BYTES or nsets * set_bytes >= ROTATE_BYTES
    writes_hbm = (nsets if in_place else ndst) * written >= WRITE_ROTATE_BYTES
    return nsets, ndst, "hbm" if reads_hbm and writes_hbm else "cache-resident"


def run_entry(torch, B, w, op: str, mode: str, steps: int, warmup: int, sets_arg: int, dev,
              srcs, flags: int = 0):
    """Time one (workload, op, mode) on the GPU; returns its entry and the
    host copy of set 0's output (the reduction's dst, or the first buffer
    after the in-place modes)."""
    stream = torch.cuda.current_stream(dev)
    src_t = [torch.from_numpy(s.view(np.uint8)).to(dev) for s in srcs]
    buf_bytes = w.buffer_elems * w.esize
    dst_t = torch.full((buf_bytes,), 0xFF, dtype=torch.uint8, device=dev)
    dt, opc = B.DTYPES[w.dtype], B.OPS[op]
    algo_bytes = algorithmic_bytes(w, mode)
    # Every step reads from and writes to HBM: when one set of buffers fits
    # in the Infinity Cache the steps rotate over copies of it, and the
    # buffers a step writes -- dst, or the sources themselves for the
    # in-place modes -- rotate until WRITE_ROTATE_BYTES are written between
    # two uses of one.  --sets S instead takes exactly S sets and S dsts.
    in_place = mode in ("allreduce", "reduce_scatter_ring")
    nsets, ndst, residency = rotation(w, mode, sets_arg)
    sets = [src_t] + [[t.clone() for t in src_t] for _ in range(nsets - 1)]
    dsts = [dst_t] + [dst_t.clone() for _ in range(ndst - 1)]
    # host pointer arrays built once, so the timed calls marshal only scalars
    set_ptrs = [B.pointer_array([t.data_ptr() for t in srcs_k]) for srcs_k in sets]
    dst_ptrs = [dst_k.data_ptr() for dst_k in dsts]
    cuda_stream = stream.cuda_stream
    tuning = B.tuning(flags=flags) if flags else None
    launches, launch = 1, None
    if mode == "treduce":
        st, info = B.ptored_treduce_plan([t.data_ptr() for t in src_t], w.nranks, w.root,
                                         dst_t.data_ptr(), w.rows, w.cols, w.ld, w.valid_rows,
                                         w.valid_cols, dt, opc, tuning)
        if st != 0:
            raise RuntimeError(B.ptored_status_string(st))
        launches = int(info.launches)
        # how the library launches the call (its own plan, no HIP call)
        launch = {"kernel_family": B.PATHS[info.path],
                  "walk": {0: "contiguous", 1: "row_tiles", 2: "flattened"}[info.rows_mode],
                  "workgroup_threads": B.PTORED_WORKGROUP_THREADS,
                  "slots_per_thread": int(info.slots_per_thread),
                  "workgroups_per_cu": int(info.wgs_per_cu) or "all that fit",
                  "lead_bytes": int(info.lead), "launches": launches}

    def call(step_no):
        k, kd = step_no % nsets, step_no % ndst
        ptrs = set_ptrs[k]
        if mode == "treduce":
            if tuning is not None:
                return B.ptored_treduce_ex(ptrs, w.nranks, w.root, dst_ptrs[kd], w.rows, w.cols,
                                           w.ld, w.valid_rows, w.valid_cols, dt, opc, tuning,
                                           cuda_stream)
            return B.ptored_treduce(ptrs, w.nranks, w.root, dst_ptrs[kd], w.rows, w.cols,
                                    w.ld, w.valid_rows, w.valid_cols, dt, opc, cuda_stream)
        if mode == "allreduce":
            return B.ptored_allreduce(ptrs, w.nranks, w.root, w.rows, w.cols, w.ld,
                                      w.valid_rows, w.valid_cols, dt, opc, tuning, cuda_stream)
        if mode == "reduce_scatter_ring":  # in place: segment s back into rank s's buffer
            return B.ptored_reduce_scatter_ring(ptrs, w.nranks, ptrs, w.buffer_elems, dt, opc,
                                                tuning, cuda_stream)
        if mode == "accumulate_add":
            return B.ptored_accumulate_add(ptrs, w.nranks, dst_ptrs[kd], w.rows, w.cols,
                                           w.ld, w.valid_rows, w.valid_cols, dt, tuning,
                                           cuda_stream)
        dsts[kd].copy_(sets[k][0])  # memcpy: the runtime's device-to-device copy
        return 0

    nstep = [0]

    def step():
        st = call(nstep[0])
        nstep[0] += 1
        if st != 0:
            raise RuntimeError(B.ptored_status_string(st))

    ms_step, per_step = time_steps(torch, stream, step, steps, warmup)
    gbs = algo_bytes / (ms_step * 1e-3) / 1e9
    out = dst_t if mode in ("treduce", "accumulate_add", "memcpy") else src_t[0]
    host_out = out.cpu().numpy().view(W_STORAGE[w.dtype])
    entry = {
        "workload": w.name, "op": op, "mode": mode, "nranks": w.nranks, "dtype": w.dtype,
        "rows": w.rows, "cols": w.cols, "ld": w.ld, "valid_rows": w.valid_rows,
        "valid_cols": w.valid_cols, "root": w.root, "values": w.recipe,
        "algorithmic_bytes_per_step": algo_bytes, "launches_per_step": launches,
        "input_sets": nsets, "dst_buffers": None if in_place else ndst,
        "residency": residency, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 5),
                    "min": round(per_step[0], 5), "max": round(per_step[-1], 5)},
        "gbs": round(gbs, 2),
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "elements_per_s": round(w.valid_rows * w.valid_cols / (ms_step * 1e-3), 1),
        "launch": launch,
        "tuning_flags": flags,
        "traffic": (stored_traffic(w.name, op, mode) if mode != "memcpy" and not flags
                    else None),
    }
    del sets, dsts, src_t, dst_t, out
    torch.cuda.empty_cache()
    return entry, host_out


W_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16, "i32": np.int32}


def _hip_runtime():
    """The HIP runtime torch mapped into this process (for hipMemcpyAsync)."""
    import ctypes

    path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
    lib = ctypes.CDLL(path)
    lib.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    lib.hipMemcpyAsync.restype = ctypes.c_int
    return lib


HIP_MEMCPY_DEVICE_TO_DEVICE = 3


def measure_ceilings(torch, B, dev, steps: int, warmup: int):
    """Practical ceilings on this device, in this process: the runtime's
    device-to-device hipMemcpyAsync of 1 GiB, and the library's own copy
    kernel (one source, the N = 1 path) over 1 GiB; 2 GiB moved per call."""
    from cross_rank_collective_amd import workloads as W

    cal = W.CALIBRATION["n1_i32_16384x16384_copy"]
    nbytes = cal.valid_bytes
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(cal.seed_base)
    a = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=g)
    b = torch.zeros_like(a)
    hip = _hip_runtime()

    def memcpy_step():
        rc = hip.hipMemcpyAsync(b.data_ptr(), a.data_ptr(), nbytes,
                                HIP_MEMCPY_DEVICE_TO_DEVICE, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyAsync returned {rc}")

    srcs = B.pointer_array([a.data_ptr()])

    def copy_step():
        st = B.ptored_treduce(srcs, 1, 0, b.data_ptr(), cal.rows, cal.cols, cal.ld,
                              cal.valid_rows, cal.valid_cols, B.DTYPES[cal.dtype],
                              B.OPS["sum"], stream.cuda_stream)
        if st != 0:
            raise RuntimeError(B.ptored_status_string(st))

    out = {}
    for name, step in (("hipMemcpyAsync_d2d_1GiB", memcpy_step),
                       ("library_copy_kernel_1GiB", copy_step)):
        b.zero_()
        ms, per = time_steps(torch, stream, step, steps, warmup)
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bytes_per_call": 2 * nbytes, "ms_per_call": round(ms, 5),
                     "gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "bitwise_copy": bool(torch.equal(a, b))}
    del a, b
    torch.cuda.empty_cache()
    return out


def device_identity(torch, dev) -> dict:
    p = torch.cuda.get_device_properties(dev)
    arch = getattr(p, "gcnArchName", "?")
    return {"name": p.name or arch.split(":")[0], "arch": arch,
            "uuid": str(getattr(p, "uuid", "?")),
            "pci": f"{getattr(p, 'pci_domain_id', 0):04x}:{getattr(p, 'pci_bus_id', 0):02x}:"
                   f"{getattr(p, 'pci_device_id', 0):02x}",
            "compute_units": p.multi_processor_count, "memory_bytes": p.total_memory,
            "host": platform.node()}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200, or 1000 for a workload whose step "
                         "moves less than 64 MiB, whose launches are short and noisy)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--op", default=None)
    ap.add_argument("--mode", default="treduce", choices=MODES)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (the oracle's timing and the bit-exact checks)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the named workload (no other configs, no ceilings)")
    ap.add_argument("--flags", type=lambda x: int(x, 0), default=0,
                    help="ptored tuning flags of the named workload's calls (PTORED_* bits, "
                         "e.g. 0x200 = per-rank push-with-add); 0 = automatic")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets and dsts the steps rotate over (0 = automatic: input "
                         "sets rotated when one set fits in the Infinity Cache, and the "
                         "buffers a step writes rotated until 512 MiB are written between "
                         "two uses of one, so that every step reads from and writes to HBM)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM-traffic summaries from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="write the kernel-trace summaries from a rocprofv3 --kernel-trace "
                         "--stats run (with --bench-log: the bench output of that run)")
    ap.add_argument("--bench-log", default=None)
    ap.add_argument("--commands", nargs="*", default=[],
                    help="the rocprofv3 commands, recorded in the summaries")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args)
    if args.summarize_trace:
        return summarize_trace(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the reduction; runs on more than one GPU "
              "are not supported (use --gpus 1)", file=sys.stderr)
        return 2

    import torch

    from cross_rank_collective_amd import binding as B
    from cross_rank_collective_amd import workloads as W

    name = args.workload or W.HEADLINE
    w = W.find(name)
    op = args.op or w.ops[0]
    mode = args.mode
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load()
    cpu_leg = not args.no_cpu_baseline

    def steps_for(wk, md):
        if args.steps is None:
            return 1000 if algorithmic_bytes(wk, md) < SMALL_STEP_BYTES else 200
        # other entries than the headline: short launches are timed over at
        # least 1000 steps whatever K is
        return args.steps

    steps = steps_for(w, mode)
    srcs = W.make_sources(w)
    head, head_out = run_entry(torch, B, w, op, mode, steps, args.warmup, args.sets, dev, srcs,
                               args.flags)

    line = {
        "metric": METRIC[mode],
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "step_ms": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {k: head[k] for k in (
            "workload", "op", "nranks", "rows", "cols", "ld", "valid_rows", "valid_cols",
            "root", "values", "mode", "algorithmic_bytes_per_step", "launches_per_step",
            "input_sets", "dst_buffers", "residency")},
        "launch": head["launch"],
        "tuning_flags": args.flags,
        "pct_of_peak": round(100.0 * head["gbs"] / HBM_PEAK_GBS, 2),
        "elements_per_s": head["elements_per_s"],
        "roofline": {
            "bound": "hbm",
            "achieved": head["gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": head["frac"],
            "traffic": head["traffic"],
            "kernel": MODE_KERNEL[mode],
            "kernel_source_hash": kernel_source_hash(),
        },
        "device": device_identity(torch, dev),
    }
    if cpu_leg and mode == "treduce":
        line["gpu_bit_exact"] = oracle_full_check(w, op, srcs, head_out)
        line["cpu_baseline"] = cpu_baseline(w, op, srcs, head_out)
    if mode == "treduce" and not args.headline_only:
        configs = {}
        cache = {w.name: srcs}
        for wl, o in default_run():
            if (wl, o) == (w.name, op):
                continue
            wk = W.find(wl)
            if wk.name not in cache:
                cache.clear()
                cache[wk.name] = W.make_sources(wk)
            k = steps_for(wk, mode)
            if algorithmic_bytes(wk, mode) < SMALL_STEP_BYTES:
                k = max(k, 1000)
            entry, out = run_entry(torch, B, wk, o, mode, k, args.warmup, 0, dev,
                                   cache[wk.name])
            if cpu_leg:
                entry["gpu_bit_exact"] = oracle_full_check(wk, o, cache[wk.name], out)
            configs[f"{wl}:{o}"] = entry
            del out
        cache.clear()
        line["configs"] = configs
    if not args.headline_only:
        line["ceilings"] = measure_ceilings(torch, B, dev, max(steps, 20), args.warmup)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
