"""GPU: the entry points recorded in a HIP graph and replayed, and called
from several host threads at once.

Graph capture: the reduction (a launch with the resident-workgroup limit,
and a ragged 2-D one with row tiles and tail tiles), the in-place allreduce,
the ring reduce-scatter and push-with-add are captured once with
torch.cuda.graph and replayed three times, with new inputs written by eager
work between the replays.  Every replay must equal the same call made eagerly on the same
inputs, bit for bit over the whole output, and sampled rows must equal the
oracle.  The library records no memset and allocates nothing, so nothing
it issues is out of place in a graph.

Threads: four host threads, each with its own stream and buffers, call the
library concurrently (the binding releases the interpreter lock); every
result must equal the oracle.  And four host threads on their own streams
push-with-add into one shared dst at the same time: with sums that are
exact in any order, the result must be dst plus every push.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from cross_rank_collective_amd import binding as B
from tests.gpu_helpers import compare, say, sentinel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _bf16(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32) * np.float32(0.01))
    return x.to(torch.bfloat16)


def _oracle_rows(srcs, dtype, op, root, rows_idx, cols, ld, vc):
    """The oracle's result on the given rows (each folded as a 1 x vc row)."""
    out = []
    for r in rows_idx:
        ins = [np.ascontiguousarray(s[r * ld:r * ld + vc]) for s in srcs]
        want = sentinel(dtype, vc)
        oracle.treduce(ins, want, root=root, dtype=dtype, op=op, rows=1, cols=vc, ld=vc,
                       valid_rows=1, valid_cols=vc)
        out.append(want)
    return out


def _host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def test_graph_capture_and_replay():
    rng = np.random.default_rng(91)
    n, rows, cols = 8, 2048, 4096            # 4096 tiles: the resident limit applies
    rr, rc, rld, rvr, rvc = 700, 1798, 1800, 699, 1797  # ragged 2-D: row tiles + tail tiles
    srcs = [_bf16(rng, (rows, cols)).cuda() for _ in range(n)]
    rsrcs = [_bf16(rng, (rr, rld)).cuda() for _ in range(n)]
    dst = torch.full((rows, cols), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    rdst = torch.full((rr, rld), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    bufs = [_bf16(rng, (rows, cols)).cuda() for _ in range(4)]       # allreduce, in place
    ring_src = [_bf16(rng, (rows * cols,)).cuda() for _ in range(4)]
    ring_dst = [torch.full((rows * cols,), -1, dtype=torch.int16,
                           device="cuda").view(torch.bfloat16) for _ in range(4)]
    acc_src = [_bf16(rng, (rr, rld)).cuda() for _ in range(3)]   # push-with-add, ragged
    acc_dst = _bf16(rng, (rr, rld)).cuda()
    dt, sum_, mx = B.DTYPES["bf16"], B.OPS["sum"], B.OPS["max"]

    def calls(stream):
        st = [B.ptored_treduce([t.data_ptr() for t in srcs], n, 3, dst.data_ptr(), rows, cols,
                               cols, rows, cols, dt, sum_, stream),
              B.ptored_treduce([t.data_ptr() for t in rsrcs], n, 0, rdst.data_ptr(), rr, rc, rld,
                               rvr, rvc, dt, mx, stream),
              B.ptored_allreduce([t.data_ptr() for t in bufs], 4, 1, rows, cols, cols, rows, cols,
                                 dt, sum_, None, stream),
              B.ptored_reduce_scatter_ring([t.data_ptr() for t in ring_src], 4,
                                           [t.data_ptr() for t in ring_dst], rows * cols, dt,
                                           sum_, None, stream),
              B.ptored_accumulate_add([t.data_ptr() for t in acc_src], 3, acc_dst.data_ptr(),
                                      rr, rc, rld, rvr, rvc, dt, None, stream)]
        assert st == [0, 0, 0, 0, 0], st

    def fresh_inputs(seed):
        g = np.random.default_rng(seed)
        for t in srcs + bufs:
            t.copy_(_bf16(g, (rows, cols)))
        for t in rsrcs:
            t.copy_(_bf16(g, (rr, rld)))
        for t in ring_src:
            t.copy_(_bf16(g, (rows * cols,)))
        for t in acc_src + [acc_dst]:
            t.copy_(_bf16(g, (rr, rld)))

    def snapshot():
        return [dst.clone(), rdst.clone()] + [b.clone() for b in bufs] + \
               [d.clone() for d in ring_dst] + [acc_dst.clone()]

    calls(torch.cuda.current_stream().cuda_stream)  # warm the per-device caches
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph replay {rep}")
        fresh_inputs(100 + rep)
        keep = [b.clone() for b in bufs + [acc_dst]]
        host_srcs = [_host_bits(t) for t in srcs]
        host_rsrcs = [_host_bits(t) for t in rsrcs]
        host_acc = [_host_bits(t) for t in acc_src + [acc_dst]]
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        # the same calls made eagerly on the same inputs
        for b, k in zip(bufs + [acc_dst], keep):
            b.copy_(k)
        calls(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        want = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rep, i)
        # sampled rows against the oracle
        pick = [0, rows - 1, int(rng.integers(0, rows))]
        ref = _oracle_rows(host_srcs, "bf16", "sum", 3, pick, cols, cols, cols)
        d = _host_bits(got[0])
        for r, w in zip(pick, ref):
            assert compare("bf16", d[r * cols:(r + 1) * cols], w).all(), (rep, r)
        pick = [0, rvr - 1, int(rng.integers(0, rvr))]
        ref = _oracle_rows(host_rsrcs, "bf16", "max", 0, pick, rc, rld, rvc)
        d = _host_bits(got[1])
        for r, w in zip(pick, ref):
            assert compare("bf16", d[r * rld:r * rld + rvc], w).all(), (rep, r)
            assert np.all(d[r * rld + rvc:(r + 1) * rld] == 0xFFFF)  # outside valid: untouched
        # push-with-add: dst + fold of its sources (rank order), rounded once
        want = host_acc[3].copy()
        fold = sentinel("bf16", want.size)
        oracle.treduce(host_acc[:3], fold, root=0, dtype="bf16", op="sum", rows=rr, cols=rc,
                       ld=rld, valid_rows=rvr, valid_cols=rvc)
        m = np.zeros((rr, rld), dtype=bool)
        m[:rvr, :rvc] = True
        m = m.reshape(-1)
        want[m] = oracle.combine_bits("bf16", "sum", want[m].astype(np.uint32),
                                      fold[m].astype(np.uint32)).astype(np.uint16)
        assert compare("bf16", _host_bits(got[-1]), want).all(), rep


def test_concurrent_host_threads():
    def worker(k):
        rng = np.random.default_rng(200 + k)
        stream = torch.cuda.Stream()
        n, rows, cols, ld = 4 + k, 300 + 37 * k, 257 + 11 * k, 264 + 11 * k
        dtype = ["f32", "i32", "f32", "i32"][k]
        op = ["sum", "max", "min", "sum"][k]
        size = (rows - 1) * ld + cols
        if dtype == "f32":
            host = [rng.standard_normal(size).astype(np.float32) for _ in range(n)]
        else:
            host = [rng.integers(-2 ** 20, 2 ** 20, size, dtype=np.int32) for _ in range(n)]
        with torch.cuda.stream(stream):
            dev = [torch.from_numpy(h).cuda() for h in host]
            out = torch.full((size,), -1, dtype=torch.int32, device="cuda")
            for it in range(20):
                st = B.ptored_treduce([t.data_ptr() for t in dev], n, it % n, out.data_ptr(),
                                      rows, cols, ld, rows - 1, cols - 2, B.DTYPES[dtype],
                                      B.OPS[op], stream.cuda_stream)
                assert st == 0
            stream.synchronize()
            got = out.cpu().numpy().view(host[0].dtype)
        want = sentinel(dtype, size)
        oracle.treduce(host, want, root=19 % n, dtype=dtype, op=op, rows=rows, cols=cols, ld=ld,
                       valid_rows=rows - 1, valid_cols=cols - 2)
        return bool(compare(dtype, got, want).all())

    say("four host threads")
    with ThreadPoolExecutor(4) as ex:
        assert all(ex.map(worker, range(4)))


@pytest.mark.parametrize("dtype", ["i32", "f16"])
def test_concurrent_pushes_into_one_dst(dtype):
    """Four host threads, each on its own stream, push-with-add into the same
    dst at the same time, several times each (both paths).  The values are
    small integers, so every order of the additions gives the same exact
    sum: dst must end as d0 plus every push, none lost."""
    rng = np.random.default_rng(300 if dtype == "i32" else 301)
    rows, cols, ld, n, reps = 257, 1000, 1024, 3, 5
    size = (rows - 1) * ld + cols
    m = np.zeros((rows, ld), dtype=bool)
    m[:, :cols] = True
    m = m.reshape(-1)[:size]

    def draw(k):
        if dtype == "i32":
            return rng.integers(-1000, 1000, size).astype(np.int32)
        return rng.integers(-2, 3, size).astype(np.float16).view(np.uint16)

    d0 = draw(0)
    dst = torch.from_numpy(d0.view(np.uint8).copy()).cuda()
    pushes = [[draw(1) for _ in range(n)] for _ in range(4)]
    dev = [[torch.from_numpy(p.view(np.uint8).copy()).cuda() for p in ps] for ps in pushes]
    torch.cuda.synchronize()

    def worker(k):
        stream = torch.cuda.Stream()
        flags = B.PTORED_ACC_PER_RANK if k % 2 else 0
        for _ in range(reps):
            st = B.ptored_accumulate_add([t.data_ptr() for t in dev[k]], n, dst.data_ptr(), rows,
                                         cols, ld, rows, cols, B.DTYPES[dtype],
                                         B.tuning(flags=flags), stream.cuda_stream)
            assert st == 0
        stream.synchronize()
        return True

    say(f"four threads pushing into one dst ({dtype})")
    with ThreadPoolExecutor(4) as ex:
        assert all(ex.map(worker, range(4)))
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(d0.dtype)
    if dtype == "i32":
        total = d0.astype(np.int64) + reps * sum(p.astype(np.int64) for ps in pushes for p in ps)
        want = np.where(m, total, d0.astype(np.int64)).astype(np.int32)
    else:
        vals = d0.view(np.float16).astype(np.float64) + reps * sum(
            p.view(np.float16).astype(np.float64) for ps in pushes for p in ps)
        want = np.where(m, vals.astype(np.float16).view(np.uint16), d0)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
