"""GPU parity of the bucketed all-reduce and the tensor-parallel layouts
(all-gather and reduce-scatter along dim 1) against the CPU oracle; calls go
through the C ABI.  Every comparison is bit for bit: the bucket folds each
element in the ring order of its bucket chunk, and feature slice c of the
reduce-scatter in the ring order of chunk c, exactly as the oracle does.
"""

import numpy as np
import pytest

import oracle_pins as PIN
import workloads as W
from gpu_util import assert_bitwise, to_dev, to_host
from oracle import collectives as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DTYPES = ("int32", "float32", "bfloat16", "float16")


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def ops_for(dtype):
    return ("sum", "max", "min") + (("avg",) if dtype != "int32" else ())


def run_bucket(rr, parts, dtype, op, in_place=False):
    devs = [to_dev(t, dtype) for t in parts]
    outs = None if in_place else [torch.empty_like(d) for d in devs]
    res = rr.all_reduce_bucket(devs, outs, op=op)
    return [np.stack([to_host(x, dtype) for x in r]) for r in res]


def check_bucket(got, want, what):
    assert len(got) == len(want)
    for i, (g, w) in enumerate(zip(got, want)):
        assert_bitwise(g, w, f"{what}: tensor {i}")


# ---------------------------------------------------------------------------
# Bucketed all-reduce.

def test_bucket_ring_probe(rr):
    """The ring-order probe cut into tensors still folds every element in its
    bucket chunk's order (all zeros)."""
    x = PIN.enc(PIN.ring_order_probe_inputs(), "float32")
    for cut in ((1, 3), (2, 2), (3, 1), (1, 1, 1, 1)):
        parts, o = [], 0
        for w in cut:
            parts.append(np.ascontiguousarray(x[:, o:o + w]))
            o += w
        got = run_bucket(rr, parts, "float32", "sum")
        check_bucket(got, C.all_reduce_bucket(parts, "sum", "float32"), f"cut {cut}")
        for g in got:
            assert not np.any(g), cut


BUCKET_CASES = [
    (1, [5, 0, 7]),
    (2, [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]),
    (3, [4099, 1, 0, 65536 + 12, 3]),
    (8, [768 * 64, 768, 768, 64 * 3072, 3072, 1, 77777]),
    (8, [int(v) for v in np.random.default_rng(0).integers(0, 3000, size=300)]),  # many launches
    (64, [200000, 33, 64 * 64 + 5]),  # more pieces than one launch holds
    (16, [0, 0, 123457]),
]


@pytest.mark.parametrize("case", range(len(BUCKET_CASES)))
@pytest.mark.parametrize("dtype", DTYPES)
def test_bucket_sweep(rr, case, dtype):
    p, sizes = BUCKET_CASES[case]
    parts = [W.random_inputs(41 + i, p, n, dtype, kind="full" if dtype == "int32" else "normal")
             for i, n in enumerate(sizes)]
    for op in ops_for(dtype):
        check_bucket(run_bucket(rr, parts, dtype, op), C.all_reduce_bucket(parts, op, dtype), f"p={p} {op}")


@pytest.mark.parametrize("dtype", ("float32", "bfloat16", "float16"))
def test_bucket_unaligned_and_in_place(rr, dtype):
    """Tensors that are views at element offsets (not 16-byte aligned) next to
    aligned ones, out of place and in place."""
    p = 4
    sizes = [1001, 4096, 333, 8192 + 3]
    parts = [W.random_inputs(51 + i, p, n, dtype) for i, n in enumerate(sizes)]
    want = C.all_reduce_bucket(parts, "sum", dtype)
    store = torch.zeros((p, sum(sizes) + 8 * len(sizes) + 8), dtype=to_dev(parts[0][:1], dtype).dtype,
                        device="cuda")
    views, o = [], 1  # start one element in: every view but the aligned ones is misaligned
    for i, n in enumerate(sizes):
        off = o if i % 2 == 0 else ((o + 7) // 8) * 8
        v = store[:, off:off + n]
        v.copy_(to_dev(parts[i], dtype))
        views.append([v[r] for r in range(p)])
        o = off + n
    outs = [[torch.empty(n, dtype=store.dtype, device="cuda") for _ in range(p)] for n in sizes]
    res = rr.all_reduce_bucket(views, outs, op="sum")
    check_bucket([np.stack([to_host(x, dtype) for x in r]) for r in res], want, "unaligned views")
    rr.all_reduce_bucket(views, None, op="sum")
    check_bucket([np.stack([to_host(x, dtype) for x in r]) for r in views], want, "in place")


def test_bucket_gpt2_block_full_size(rr):
    """The gradients of one GPT-2-small block (12 tensors, 27 MiB per rank)
    as one bucket, every element compared; AVG as DDP uses it."""
    parts = W.bucket_inputs("gpt2_block_fp32_p8")
    for op in ("avg", "sum"):
        check_bucket(run_bucket(rr, parts, "float32", op), C.all_reduce_bucket(parts, op, "float32"), op)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", ("0", "1"))
@pytest.mark.parametrize("dtype,scale", [("bfloat16", 1), ("float32", 2), ("float16", 1)])
def test_bucket_one_round_tile_sizes(rr, tuning, dtype, scale, batch):
    """One-round buckets of GPT-2 block shapes (13.5 MiB per rank): tiles of
    8 units per lane, one per workgroup, where they number between one and
    two per CU (batch 0, the default), and the tiles of 4 units (batch 1);
    every element against the oracle."""
    p = 8
    sizes = [max(8, n // scale) + 3 * i for i, n in enumerate(W.BUCKETS["gpt2_block_fp32_p8"]["sizes"])]
    parts = [W.random_inputs(101 + i, p, n, dtype) for i, n in enumerate(sizes)]
    tuning.set("RR_AR_BATCH", batch)
    for op in ("avg", "max"):
        check_bucket(run_bucket(rr, parts, dtype, op), C.all_reduce_bucket(parts, op, dtype), f"{dtype} {op}")
    torch.cuda.empty_cache()


def test_bucket_barrier(rr, tuning):
    """A bucket of several rounds separates its read and write phases with
    the soft barrier.  A 1 us bound makes the waits run out: the results must
    not change and the timeouts must be counted.  Without the barrier, and
    with more workgroups per CU requested than fit at once (the grid is
    capped at residency, so no wait runs out), the bits are the same."""
    p = 8
    sizes = [3 * (1 << 20) + 5, 1 << 22, 777]
    parts = [W.random_inputs(81 + i, p, n, "float32") for i, n in enumerate(sizes)]
    want = C.all_reduce_bucket(parts, "avg", "float32")
    t0 = rr.barrier_timeouts()
    check_bucket(run_bucket(rr, parts, "float32", "avg"), want, "default")
    assert rr.barrier_timeouts() == t0
    tuning.set("RR_MULTI_PER_CU", "64")
    check_bucket(run_bucket(rr, parts, "float32", "avg"), want, "64 workgroups per CU requested")
    assert rr.barrier_timeouts() == t0
    tuning.unset("RR_MULTI_PER_CU")
    tuning.set("RR_PHASE_SYNC", "0")
    check_bucket(run_bucket(rr, parts, "float32", "avg"), want, "no barrier")
    tuning.unset("RR_PHASE_SYNC")
    tuning.set("RR_PHASE_TIMEOUT_US", "1")
    for _ in range(2):
        check_bucket(run_bucket(rr, parts, "float32", "avg"), want, "1 us barrier bound")
    assert rr.barrier_timeouts() > t0, "the forced bound never ran out: the bucket's barrier was not exercised"
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", ("0", "1"))
@pytest.mark.parametrize("p", (5, 8))
@pytest.mark.parametrize("strips", ("1", "2", "3", "8"))
def test_bucket_interleaved_tiles(rr, tuning, strips, p, batch):
    """A multi-round bucket whose vector pieces hold whole tiles taken in runs
    of interleaved tiles (1 = contiguous), with ragged and unaligned tensors
    beside them, in batched rounds (several tiles per workgroup and round,
    one partial round here) and in single-tile rounds (batch 1): the
    oracle's bits for sum and max, and no wait runs out."""
    sizes = [3 * (1 << 20) + 5, 1 << 22, 777, 9 * 4096 + 8, (1 << 21) + 4]
    parts = [W.random_inputs(91 + i, p, n, "float32") for i, n in enumerate(sizes)]
    tuning.set("RR_PHASE_STRIPS", strips)
    tuning.set("RR_AR_BATCH", batch)
    t0 = rr.barrier_timeouts()
    for op in ("sum", "max"):
        check_bucket(run_bucket(rr, parts, "float32", op), C.all_reduce_bucket(parts, op, "float32"),
                     f"{op} strips={strips}")
    bparts = [W.random_inputs(95 + i, p, n, "bfloat16") for i, n in enumerate((1 << 23, 4099))]
    check_bucket(run_bucket(rr, bparts, "bfloat16", "avg"), C.all_reduce_bucket(bparts, "avg", "bfloat16"),
                 f"bf16 avg strips={strips}")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("per_cu", ("0", "1", "2"))
def test_bucket_batched_rounds(rr, tuning, per_cu):
    """A bucket of several batched rounds (4 tiles per workgroup and round;
    1 or 2 workgroups per CU requested, or the schedule's choice), ragged
    and unaligned tensors among large ones, float32 and bfloat16: the
    oracle's bits, and no wait runs out."""
    p = 8
    sizes = [3 * (1 << 22) + 5, 1 << 22, 777, (1 << 21) + 4]
    parts = [W.random_inputs(71 + i, p, n, "float32") for i, n in enumerate(sizes)]
    tuning.set("RR_MULTI_PER_CU", per_cu)
    t0 = rr.barrier_timeouts()
    check_bucket(run_bucket(rr, parts, "float32", "sum"), C.all_reduce_bucket(parts, "sum", "float32"), "float32")
    bparts = [W.random_inputs(75 + i, p, n, "bfloat16") for i, n in enumerate((3 * (1 << 23) + 3, 4099, 1 << 22))]
    check_bucket(run_bucket(rr, bparts, "bfloat16", "avg"), C.all_reduce_bucket(bparts, "avg", "bfloat16"), "bfloat16")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


def test_bucket_empty_and_rejected(rr):
    assert rr.all_reduce_bucket([]) == []
    a = torch.ones((4, 64), dtype=torch.int32, device="cuda")
    out = torch.full_like(a, 7)
    with pytest.raises(rr.RRError):
        rr.all_reduce_bucket([a], [out], op="avg")
    with pytest.raises(rr.RRError):  # an output overlapping another tensor's input
        rr.all_reduce_bucket([a, a[:, :8]], [out, [a[0, 8:16]] * 4])
    torch.cuda.synchronize()
    assert torch.all(out == 7)


# ---------------------------------------------------------------------------
# Tensor-parallel layouts.

TP_SHAPES = [(2, 3, 4), (4, 1, 1), (4, 7, 5), (8, 33, 64), (8, 5, 3), (3, 100, 17), (16, 9, 128), (1, 4, 8)]


@pytest.mark.parametrize("p,rows,w", TP_SHAPES)
@pytest.mark.parametrize("dtype", DTYPES)
def test_all_gather_dim1(rr, p, rows, w, dtype):
    sh = W.random_inputs(61, p, rows * w, dtype, kind="full" if dtype == "int32" else "normal").reshape(p, rows, w)
    dev = to_dev(sh, dtype)
    out = torch.empty((p, rows, p * w), dtype=dev.dtype, device="cuda")
    rr.all_gather_dim1(dev, out)
    assert_bitwise(to_host(out, dtype), C.all_gather_dim1(sh), "all_gather_dim1")


@pytest.mark.parametrize("xcd", ("1", "2", "4"))
@pytest.mark.parametrize("p,rows,w,dtype", [(8, 33, 64, "float32"), (16, 9, 128, "bfloat16"), (4, 7, 8, "bfloat16"),
                                            (3, 100, 12, "float32"), (8, 1, 4, "int32"), (5, 301, 40, "float16")])
def test_all_gather_dim1_xcd_layout(rr, tuning, xcd, p, rows, w, dtype):
    """The XCD layout of the dim-1 all-gather (4 KiB output blocks, 1, 2 or 4
    destinations per workgroup, partial last block), forced at small
    shapes: the same bits as the oracle."""
    tuning.set("RR_FANOUT_XCD", xcd)
    sh = W.random_inputs(63, p, rows * w, dtype, kind="full" if dtype == "int32" else "normal").reshape(p, rows, w)
    dev = to_dev(sh, dtype)
    out = torch.empty((p, rows, p * w), dtype=dev.dtype, device="cuda")
    rr.all_gather_dim1(dev, out)
    assert_bitwise(to_host(out, dtype), C.all_gather_dim1(sh), f"all_gather_dim1 xcd={xcd}")


@pytest.mark.parametrize("p,rows,w", TP_SHAPES)
@pytest.mark.parametrize("dtype", DTYPES)
def test_reduce_scatter_dim1(rr, p, rows, w, dtype):
    x = W.random_inputs(62, p, rows * p * w, dtype, kind="full" if dtype == "int32" else "normal")
    x = x.reshape(p, rows, p * w)
    dev = to_dev(x, dtype)
    out = torch.empty((p, rows, w), dtype=dev.dtype, device="cuda")
    for op in ops_for(dtype):
        rr.reduce_scatter_dim1(dev, out, op=op)
        assert_bitwise(to_host(out, dtype), C.reduce_scatter_cols(x, op, dtype), f"reduce_scatter_dim1 {op}")


def test_reduce_scatter_dim1_ring_probe(rr):
    """The ring probe laid along the feature dimension, in one row and in two."""
    probe = PIN.ring_order_probe_inputs().astype(np.float32)
    for x in (probe[:, None, :], np.stack([probe, probe], axis=1)):
        x = np.ascontiguousarray(x)
        dev = to_dev(x, "float32")
        out = torch.empty((4, x.shape[1], 1), dtype=torch.float32, device="cuda")
        rr.reduce_scatter_dim1(dev, out)
        got = to_host(out, "float32")
        assert_bitwise(got, C.reduce_scatter_cols(x, "sum", "float32"), "probe")
        assert not np.any(got)


def test_tp_layouts_full_size(rr):
    """Row-parallel partial outputs of shape (8, 2048, 4096) bf16 per rank as
    [16384, 4096] matrices: reduce-scatter along dim 1 to [16384, 512] slices,
    then all-gather them back along dim 1; every element compared."""
    spec = W.WORKLOADS["tp_rowparallel_bf16_p8"]
    p = spec["p"]
    rows, cols = 8 * 2048, 4096
    x = W.make_inputs("tp_rowparallel_bf16_p8").reshape(p, rows, cols)
    want = C.reduce_scatter_cols(x, "sum", "bfloat16")
    dev = to_dev(x, "bfloat16")
    sh = torch.empty((p, rows, cols // p), dtype=torch.bfloat16, device="cuda")
    rr.reduce_scatter_dim1(dev, sh)
    assert_bitwise(to_host(sh, "bfloat16"), want, "reduce_scatter_dim1 full size")
    rr.all_gather_dim1(sh, dev)
    got = to_host(dev, "bfloat16")
    del dev, sh
    torch.cuda.empty_cache()
    full = np.concatenate([want[c] for c in range(p)], axis=1)
    for r in range(p):
        assert_bitwise(got[r], full, f"all_gather_dim1 rank {r}")


def test_tp_layouts_reject_bad_shapes(rr):
    a = torch.ones((4, 3, 10), dtype=torch.float32, device="cuda")
    out = torch.empty((4, 3, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        rr.reduce_scatter_dim1(a, out)  # 10 is not divisible by 4
    L = rr.lib()
    ptrs = rr._ptr_array([t.data_ptr() for t in a])
    optrs = rr._ptr_array([t.data_ptr() for t in out])
    assert L.rr_reduce_scatter_dim1(ptrs, optrs, 4, 3, 10, 1, 0, None) == 1
    assert L.rr_all_gather_dim1(optrs, ptrs, 4, 3, 10, 1, None) == 1
