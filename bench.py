"""Benchmark of the N-way reduction on one MI355X.

One step = one ptored_treduce call over the whole workload (every source
read once, dst written once), inputs resident in HBM.  Prints ONE JSON line:
effective HBM GB/s = (N+1) * valid bytes / time, with the roofline of the
reduce kernel and the CPU oracle timed on a bounded sample as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--op OP]
                    [--mode treduce|allreduce|reduce_scatter_ring|accumulate_add|memcpy]
                    [--sets S]

The default mode is the reduction itself (dst = fold of the N sources); the
other modes time the collective variants on the same workload: the in-place
allreduce (N reads + N writes per valid element), the ring reduce-scatter
share over the whole buffer as one stream (N reads + 1 write per element)
and push-with-add by atomics (N source reads + one read and one write of dst
per element, the least any order of the additions must move); memcpy times
the runtime's device-to-device copy of one buffer, as a context ceiling.

Steps default to 200 timed calls after W warm-up calls, and to 1000 for a
workload whose step moves less than 64 MiB (the two small ones), whose
launches last a few microseconds.

When one set of input and output buffers fits in the 256 MB Infinity Cache,
the steps rotate over enough copies of it (``--sets``, default automatic) to
touch at least 1 GiB between two uses of a set, so the figure is an HBM one;
``config.residency`` says which it is.
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
SMALL_STEP_BYTES = 64 << 20  # steps moving less than this are timed 1000 times by default
MAX_SETS = 64
# The kernel each mode launches (one launch per call at the bench's sizes).
MODE_KERNEL = {"treduce": "treduce_kernel", "allreduce": "treduce_kernel",
               "reduce_scatter_ring": "ring_kernel", "accumulate_add": "accumulate_kernel",
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
        if fn.endswith((".cuh", ".hip", ".h", ".cpp")):
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


def _counter_mean_kib(directory: str, counter: str, kernel: str = "treduce_kernel") -> float:
    """Mean per-dispatch value of one counter for one kernel, from a
    rocprofv3 --pmc run written with -f csv under `directory`."""
    import csv
    import glob

    vals = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if kernel in row.get("Kernel_Name", "") and \
                        row.get("Counter_Name") == counter:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise RuntimeError(f"no {counter} rows for {kernel} under {directory}")
    return sum(vals) / len(vals)


def summarize_counters(args) -> int:
    """Write the HBM-traffic summary of one workload from four rocprofv3 runs:
    FETCH_SIZE and WRITE_SIZE of the workload and of the 1 GiB copy."""
    from cross_rank_collective_amd import workloads as W

    w = W.find(args.workload or W.HEADLINE)
    op = args.op or w.ops[0]
    kernel = MODE_KERNEL[args.mode]
    algo = algorithmic_bytes(w, args.mode)
    cal = W.CALIBRATION["n1_i32_16384x16384_copy"]
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = args.summarize_counters
    fetch = _counter_mean_kib(fetch_dir, "FETCH_SIZE", kernel)
    write = _counter_mean_kib(write_dir, "WRITE_SIZE", kernel)
    cal_fetch = _counter_mean_kib(cal_fetch_dir, "FETCH_SIZE")
    cal_write = _counter_mean_kib(cal_write_dir, "WRITE_SIZE")
    copy_bytes = cal.valid_bytes
    fetch_scale = copy_bytes / (cal_fetch * 1024.0)
    write_scale = copy_bytes / (cal_write * 1024.0)
    traffic = fetch * 1024.0 * fetch_scale + write * 1024.0 * write_scale
    lines = [
        f"# HBM traffic per launch of {kernel}, workload {w.name}, op {op}, mode {args.mode}",
        "# from rocprofv3 counters (KiB per dispatch), scaled by a 1 GiB copy",
        f"# ({cal.name}: {copy_bytes} bytes read and written per dispatch).",
        "# commands (each its own run):",
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
    out = args.counters_out or traffic_path(w.name, op, args.mode)
    with open(out, "w") as fh:
        fh.write(text)
    print(text, end="")
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets the steps rotate over (0 = enough to defeat the "
                         "Infinity Cache when one set fits in it)")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the HBM-traffic summary from four rocprofv3 --pmc runs")
    ap.add_argument("--counters-out", default=None)
    ap.add_argument("--commands", nargs="*", default=[],
                    help="the rocprofv3 commands, recorded in the summary")
    args = ap.parse_args()
    if args.summarize_counters:
        return summarize_counters(args)

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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.load()

    srcs = W.make_sources(w)
    src_t = [torch.from_numpy(s.view(np.uint8)).to(dev) for s in srcs]
    dst_t = torch.full((w.buffer_elems * w.esize,), 0xFF, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    dt, opc = B.DTYPES[w.dtype], B.OPS[op]
    mode = args.mode
    algo_bytes = algorithmic_bytes(w, mode)
    if args.steps is None:
        args.steps = 1000 if algo_bytes < SMALL_STEP_BYTES else 200
    # Input sets: when one set of buffers fits in the Infinity Cache, the
    # steps rotate over copies so that every step reads from HBM.
    set_bytes = (2 if mode == "memcpy" else w.nranks + 1) * w.buffer_elems * w.esize
    nsets = args.sets
    if nsets <= 0:
        nsets = 1 if set_bytes >= MALL_BYTES else min(MAX_SETS, -(-ROTATE_BYTES // set_bytes))
    sets = [(src_t, dst_t)] + [([t.clone() for t in src_t], dst_t.clone())
                               for _ in range(nsets - 1)]
    # host pointer arrays built once, so the timed calls marshal only scalars
    set_ptrs = [B.pointer_array([t.data_ptr() for t in srcs_k]) for srcs_k, _ in sets]
    dst_ptrs = [dst_k.data_ptr() for _, dst_k in sets]
    cuda_stream = stream.cuda_stream
    residency = "hbm" if nsets * set_bytes >= ROTATE_BYTES else "cache-resident"
    launches = 1
    launch = None
    if mode == "treduce":
        st, info = B.ptored_treduce_plan([t.data_ptr() for t in src_t], w.nranks, w.root,
                                         dst_t.data_ptr(), w.rows, w.cols, w.ld, w.valid_rows,
                                         w.valid_cols, dt, opc)
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

    def call(k):
        srcs_k, dst_k = sets[k]
        ptrs = set_ptrs[k]
        if mode == "treduce":
            return B.ptored_treduce(ptrs, w.nranks, w.root, dst_ptrs[k], w.rows, w.cols,
                                    w.ld, w.valid_rows, w.valid_cols, dt, opc, cuda_stream)
        if mode == "allreduce":
            return B.ptored_allreduce(ptrs, w.nranks, w.root, w.rows, w.cols, w.ld,
                                      w.valid_rows, w.valid_cols, dt, opc, None, cuda_stream)
        if mode == "reduce_scatter_ring":  # in place: segment s back into rank s's buffer
            return B.ptored_reduce_scatter_ring(ptrs, w.nranks, ptrs, w.buffer_elems, dt, opc,
                                                None, cuda_stream)
        if mode == "accumulate_add":
            return B.ptored_accumulate_add(ptrs, w.nranks, dst_ptrs[k], w.rows, w.cols,
                                           w.ld, w.valid_rows, w.valid_cols, dt, None,
                                           cuda_stream)
        dst_k.copy_(srcs_k[0])  # memcpy: the runtime's device-to-device copy
        return 0

    nstep = [0]

    def step():
        st = call(nstep[0] % nsets)
        nstep[0] += 1
        if st != 0:
            raise RuntimeError(B.ptored_status_string(st))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize(dev)
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    # Per-step distribution, from a second pass with an event pair around
    # every step (not part of `value`, which is the run above).
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    for a_ev, b_ev in marks:
        a_ev.record(stream)
        step()
        b_ev.record(stream)
    torch.cuda.synchronize(dev)
    per_step = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in marks)
    gbs = algo_bytes / (ms_step * 1e-3) / 1e9
    elems_s = w.valid_rows * w.valid_cols / (ms_step * 1e-3)

    traffic = stored_traffic(name, op, mode) if mode != "memcpy" else None
    line = {
        "metric": METRIC[mode],
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 5),
                    "min": round(per_step[0], 5), "max": round(per_step[-1], 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": name, "op": op, "nranks": w.nranks, "rows": w.rows, "cols": w.cols,
            "ld": w.ld, "valid_rows": w.valid_rows, "valid_cols": w.valid_cols, "root": w.root,
            "values": w.recipe, "mode": mode, "algorithmic_bytes_per_step": algo_bytes,
            "launches_per_step": launches, "input_sets": nsets, "residency": residency,
        },
        "launch": launch,
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "elements_per_s": round(elems_s, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": MODE_KERNEL[mode],
            "kernel_source_hash": kernel_source_hash(),
        },
    }
    if not args.no_cpu_baseline and mode == "treduce":
        gpu_bits = dst_t.cpu().numpy().view(W.STORAGE[w.dtype])
        line["cpu_baseline"] = cpu_baseline(w, op, srcs, gpu_bits)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
