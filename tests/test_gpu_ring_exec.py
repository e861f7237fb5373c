"""GPU tests of the persistent ring executor (algo "ring_persistent"): the
ring schedule of page "LLM Parallelism 基础", section "Ring AllReduce", run
by one launch whose workgroups hand chunks on through device-side step flags.
It must give the bits of the fused pass and of the oracle's literal ring
simulation, at full sizes, in place, on unaligned buffers; a wait forced to
time out from the host must end the launch (counted, never hung).
"""

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


def run(rr, x, dtype, op="sum", algo="ring_persistent"):
    xs = to_dev(x, dtype)
    out = torch.empty_like(xs)
    rr.all_reduce(xs, out, op=op, algo=algo)
    return to_host(out, dtype)


@pytest.mark.parametrize("name", ["ar_int32_p4_n4096", "ar_fp32_p8_8MiB", "hier_bf16_p8g4_8MiB"])
def test_workloads_match_the_literal_ring(rr, name):
    x = W.make_inputs(name)
    dtype = W.WORKLOADS[name]["dtype"]
    f0 = rr.ring_exec_failures()
    want = C.all_reduce_ring(x, "sum", dtype) if x.shape[1] <= 4096 else C.all_reduce_fold(x, "sum", dtype)
    assert_bitwise(run(rr, x, dtype), want, name)
    assert rr.ring_exec_failures() == f0


@pytest.mark.parametrize("dtype", ("float32", "bfloat16", "float16"))
def test_large_ragged(rr, dtype):
    """Chunks of unequal length and many slices per chunk, every op."""
    p, n = 8, 8 * (1 << 20) + 8 * 5 + 3
    x = W.random_inputs(81, p, n, dtype)
    f0 = rr.ring_exec_failures()
    for op in ("sum", "avg", "max"):
        assert_bitwise(run(rr, x, dtype, op), C.all_reduce_fold(x, op, dtype), op)
    assert rr.ring_exec_failures() == f0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("slices", ("1", "8", "20"))
@pytest.mark.parametrize("dtype", ("float32", "bfloat16"))
def test_slice_counts(rr, tuning, slices, dtype):
    """Fewer slices per chunk than the default (one slice: no XCD-local
    layout; 20, rounded down to a multiple of the XCD count): the same
    bits."""
    p, n = 8, 8 * (1 << 20) + 8 * 3 + 1
    x = W.random_inputs(84, p, n, dtype)
    tuning.set("RR_EXEC_SLICES", slices)
    f0 = rr.ring_exec_failures()
    assert_bitwise(run(rr, x, dtype), C.all_reduce_fold(x, "sum", dtype), f"{slices} slices")
    assert rr.ring_exec_failures() == f0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ("int32", "float32", "bfloat16"))
def test_in_place_and_unaligned(rr, dtype):
    p, n = 6, 6 * 4001 + 5
    x = W.random_inputs(82, p, n + 3, dtype, kind="full" if dtype == "int32" else "normal")
    want = C.all_reduce_fold(np.ascontiguousarray(x[:, :n]), "sum", dtype)
    xs = to_dev(np.ascontiguousarray(x[:, :n]), dtype)
    rr.all_reduce(xs, algo="ring_persistent")
    assert_bitwise(to_host(xs, dtype), want, "in place")
    base = to_dev(x, dtype)
    ins = [base[r, 1:1 + n] for r in range(p)]
    outbuf = torch.empty((p, n + 1), dtype=base.dtype, device="cuda")
    outs = [outbuf[r, 1:1 + n] for r in range(p)]
    rr.all_reduce(ins, outs, algo="ring_persistent")
    got = np.stack([to_host(o, dtype) for o in outs])
    assert_bitwise(got, C.all_reduce_fold(np.ascontiguousarray(x[:, 1:1 + n]), "sum", dtype), "unaligned")


@pytest.mark.parametrize("dtype", ("int32", "float32"))
@pytest.mark.parametrize("p,n", ((4, 100003), (8, 3 * (1 << 16) + 7)))
def test_all_gather_rereads_after_partial_sums(rr, dtype, p, n):
    """4-byte kinds fold into the outputs, so an all-gather step reads
    predecessor chunks that a reduce-scatter step read while they held
    partial sums (and, in place, that the first step read as input).  Slices
    small enough to stay in a CU's L1 between the two reads, but still laid
    out one XCD per slice: the second read must see the final values, in
    place and out of place, on every launch."""
    f0 = rr.ring_exec_failures()
    for rep in range(4):
        x = W.random_inputs(90 + rep, p, n, dtype, kind="full" if dtype == "int32" else "normal")
        want = C.all_reduce_fold(x, "sum", dtype)
        assert_bitwise(run(rr, x, dtype), want, f"out of place, launch {rep}")
        xs = to_dev(x, dtype)
        rr.all_reduce(xs, algo="ring_persistent")
        assert_bitwise(to_host(xs, dtype), want, f"in place, launch {rep}")
    assert rr.ring_exec_failures() == f0


def test_forced_timeout_ends_the_launch(rr, tuning):
    """A 1 us bound on every wait (set from the host) makes workers give up:
    the launch must end, be counted, and a following normal launch on the
    same stream must be correct."""
    p, n = 8, 8 * (1 << 20)
    x = W.random_inputs(83, p, n, "float32")
    f0 = rr.ring_exec_failures()
    tuning.set("RR_EXEC_TIMEOUT_US", "1")
    xs = to_dev(x, "float32")
    out = torch.empty_like(xs)
    for _ in range(3):
        rr.all_reduce(xs, out, algo="ring_persistent")
    torch.cuda.synchronize()
    assert rr.ring_exec_failures() > f0, "the 1 us bound never ran out"
    tuning.unset("RR_EXEC_TIMEOUT_US")
    f1 = rr.ring_exec_failures()
    rr.all_reduce(xs, out, algo="ring_persistent")
    assert_bitwise(to_host(out, "float32"), C.all_reduce_fold(x, "sum", "float32"), "after the failed launches")
    assert rr.ring_exec_failures() == f1
    torch.cuda.empty_cache()


def test_slots_pass_between_streams(rr):
    """The step flags come in 16 slots per device; a slot whose last launch
    has completed passes to another stream, so 20 streams used one after the
    other all get one (each result checked)."""
    p, n = 4, 65536 + 5
    x = W.random_inputs(88, p, n, "float32")
    want = C.all_reduce_ring(x, "sum", "float32")
    xs = to_dev(x, "float32")
    streams = [torch.cuda.Stream() for _ in range(20)]
    assert len({s.cuda_stream for s in streams}) == 20
    torch.cuda.synchronize()
    f0 = rr.ring_exec_failures()
    for i, s in enumerate(streams):
        with torch.cuda.stream(s):
            ys = torch.empty_like(xs)
            rr.all_reduce(xs, ys, algo="ring_persistent")
            s.synchronize()
            assert_bitwise(to_host(ys, "float32"), want, f"stream {i}")
    assert rr.ring_exec_failures() == f0
