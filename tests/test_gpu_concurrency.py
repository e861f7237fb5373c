"""Concurrent use of the library (calls through the C ABI).

Collectives enqueued on several streams at once may run side by side on the
GPU.  The soft barriers of the multi-round launches are kept per stream and
order no data, so they may time out when the grids cannot all be resident
(a cost in time only); the persistent executor's step flags are kept per
stream too and its waits are bounded far above the others' run time.  Every
result must equal the oracle bit for bit.  Host threads calling the library
at the same time, each on its own stream, must get the same results as
serial calls.
"""

import threading

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bitwise, to_dev, to_host
from oracle import collectives as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def test_collectives_on_concurrent_streams(rr):
    p = 8
    jobs = []
    # several rounds of the phased fold (barrier), fp32
    x1 = W.random_inputs(91, p, 8 * (1 << 20) + 40, "float32")
    jobs.append(("all_reduce fp32", x1, "float32", C.all_reduce_ring(x1, "sum", "float32"),
                 lambda xs, ys: rr.all_reduce(xs, ys)))
    # several rounds, bf16, hierarchical with wire rounding
    x2 = W.random_inputs(92, p, 16 * (1 << 20) + 3, "bfloat16")
    jobs.append(("hier wire bf16", x2, "bfloat16", C.all_reduce_hier(x2, "sum", "bfloat16", 4, wire_round=True),
                 lambda xs, ys: rr.all_reduce_hier(xs, ys, group_size=4, wire_round=True)))
    # the persistent executor
    x3 = W.random_inputs(93, p, 2 * (1 << 20) + 9, "float32")
    jobs.append(("ring_persistent fp32", x3, "float32", C.all_reduce_ring(x3, "max", "float32"),
                 lambda xs, ys: rr.all_reduce(xs, ys, op="max", algo="ring_persistent")))
    # reduce-scatter (oversubscribed grid, no barrier)
    x4 = W.random_inputs(94, p, 8 * (1 << 20), "float32")
    jobs.append(("reduce_scatter fp32", x4, "float32", C.reduce_scatter_ring(x4, "sum", "float32"),
                 lambda xs, ys: rr.reduce_scatter(xs, ys)))
    streams = [torch.cuda.Stream() for _ in jobs]
    ins = [to_dev(x, dt) for _, x, dt, _, _ in jobs]
    outs = [torch.zeros(tuple(np.asarray(w).shape), dtype=i.dtype, device="cuda")
            for (_, _, _, w, _), i in zip(jobs, ins)]
    f0 = rr.ring_exec_failures()
    torch.cuda.synchronize()
    for rep in range(2):
        for (name, _, _, _, fn), s, xs, ys in zip(jobs, streams, ins, outs):
            with torch.cuda.stream(s):
                ys.fill_(0)
                fn(xs, ys)
        torch.cuda.synchronize()
        for (name, _, dt, want, _), ys in zip(jobs, outs):
            assert_bitwise(to_host(ys, dt), np.asarray(want), f"{name}, round {rep}")
    assert rr.ring_exec_failures() == f0, "an executor wait timed out"
    torch.cuda.empty_cache()


def test_host_threads(rr):
    """Four host threads, each on its own stream and buffers, call the
    library 25 times in a row; ctypes releases the interpreter lock during the
    calls, so the library's host side runs truly concurrently."""
    p, n = 8, 3 * (1 << 20) + 17
    cases = []
    for t in range(4):
        x = W.random_inputs(95 + t, p, n, "float32")
        op = ("sum", "max", "min", "avg")[t]
        cases.append((x, op, C.all_reduce_ring(x, op, "float32")))
    errors = []

    def worker(t):
        try:
            x, op, want = cases[t]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                xs = to_dev(x, "float32")
                ys = torch.empty_like(xs)
                s.synchronize()
                algo = ("ring", "ring_staged", "ring", "ring_persistent")[t]
                for _ in range(25):
                    rr.all_reduce(xs, ys, op=op, algo=algo)
                s.synchronize()
                got = to_host(ys, "float32")
            if not np.array_equal(got.view(np.uint32), np.asarray(want).view(np.uint32)):
                errors.append(f"thread {t} ({op}): result differs from the oracle")
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(f"thread {t}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.empty_cache()
