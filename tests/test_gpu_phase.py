"""GPU tests of the phased fold that serves the fused all-reduces on aligned
buffers: shapes that take several rounds (so the soft barrier between the
read and the write phase runs), ragged chunk bounds (tiles that do not tile
the chunks, heads and tails in their own launch), p without a compiled
kernel, the bounded wait forced to time out, and a requested grid larger
than the device keeps resident.  The barrier orders no data, so every case
must match the CPU oracle bit for bit whatever the barrier does.
"""

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bitwise, to_dev, to_host
from oracle import collectives as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# (p, n): several rounds of 256-lane tiles at the default grid, with chunk
# bounds floor(c*n/p) that are not multiples of the 16-byte group.
MULTI_ROUND = [(8, 8 * (1 << 20) + 8 * 3 + 5), (5, 5 * (1 << 21) + 7)]


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def run_ar(rr, x, dtype, op, algo, group=0):
    xs = to_dev(x, dtype)
    out = torch.empty_like(xs)
    rr.all_reduce(xs, out, op=op, algo=algo, group_size=group)
    got = to_host(out, dtype)
    del xs, out
    return got


@pytest.mark.parametrize("p,n", MULTI_ROUND)
@pytest.mark.parametrize("dtype", ("int32", "float32", "bfloat16"))
def test_multi_round_ragged_ring(rr, p, n, dtype):
    if dtype == "bfloat16":
        n = 2 * n + 1  # twice the elements per 16-byte group: as many rounds
    x = W.random_inputs(61, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    t0 = rr.barrier_timeouts()
    for op in ("sum", "max"):
        assert_bitwise(run_ar(rr, x, dtype, op, "ring"), C.all_reduce_fold(x, op, dtype), f"ring {op}")
    assert rr.barrier_timeouts() == t0, "a phase barrier timed out on an otherwise idle GPU"
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ("float32", "bfloat16"))
def test_multi_round_ragged_hier(rr, dtype):
    p, n = 8, 8 * (1 << 20) * (2 if dtype == "bfloat16" else 1) + 13
    x = W.random_inputs(62, p, n, dtype)
    for G in (2, 4):
        assert_bitwise(run_ar(rr, x, dtype, "sum", "hier", G), C.all_reduce_hier(x, "sum", dtype, G),
                       f"hier G={G}")
    torch.cuda.empty_cache()


HIER_BATCH_CASES = [
    # (p, G, n, dtype, op): one partial batched round, full rounds, ragged
    # lengths, groups of 2, 3 and 4
    (8, 4, 6 << 20, "float32", "sum"),
    (8, 2, (12 << 20) + 8 * 5 + 3, "bfloat16", "max"),
    (6, 3, (5 << 20) + 7, "float32", "avg"),
    (8, 4, 20 << 20, "bfloat16", "sum"),
]


@pytest.mark.parametrize("env", [{}, {"RR_AR_BATCH": "1"}, {"RR_AR_BATCH": "2"}, {"RR_PHASE_STRIPS": "1"}])
@pytest.mark.parametrize("case", range(len(HIER_BATCH_CASES)))
def test_hier_batched_rounds(rr, tuning, env, case):
    """The hierarchical all-reduce of several rounds in batched rounds (K
    tiles per workgroup and round, interleaved runs, the write phase output
    by output) and in single-tile rounds: the oracle's bits, no wait runs
    out."""
    p, G, n, dtype, op = HIER_BATCH_CASES[case]
    x = W.random_inputs(76 + case, p, n, dtype)
    for k, v in env.items():
        tuning.set(k, v)
    t0 = rr.barrier_timeouts()
    assert_bitwise(run_ar(rr, x, dtype, op, "hier", G), C.all_reduce_hier(x, op, dtype, G), f"{p} {G} {n} {env}")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


def test_forced_barrier_timeouts_keep_results(rr, tuning):
    """A 1 us bound makes the barrier waits run out; the results must not
    change, and the timeouts must be counted."""
    p, n = 8, 8 * (1 << 20) + 40
    x = W.random_inputs(63, p, n, "float32")
    want = C.all_reduce_fold(x, "sum", "float32")
    tuning.set("RR_PHASE_TIMEOUT_US", "1")
    t0 = rr.barrier_timeouts()
    for _ in range(3):
        assert_bitwise(run_ar(rr, x, "float32", "sum", "ring"), want, "ring with 1 us barrier bound")
    assert rr.barrier_timeouts() > t0, "the forced bound never ran out: the timeout path was not exercised"
    torch.cuda.empty_cache()


def test_oversized_grid_is_capped_to_residency(rr, tuning):
    """Asking for more workgroups per compute unit than fit at once must not
    leave the barrier waiting on workgroups that cannot run."""
    p, n = 8, 8 * (1 << 21)
    x = W.random_inputs(64, p, n, "bfloat16")
    want = C.all_reduce_fold(x, "sum", "bfloat16")
    tuning.set("RR_PHASE_PER_CU", "8")
    t0 = rr.barrier_timeouts()
    assert_bitwise(run_ar(rr, x, "bfloat16", "sum", "ring"), want, "ring, 8 workgroups per CU requested")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("env", [{"RR_PHASE": "0"}, {"RR_PHASE_SYNC": "0"}, {"RR_PHASE_STATIC": "0"},
                                 {"RR_PHASE_STATIC": "1"}, {"RR_PHASE_U": "4"}, {"RR_PHASE_GRID": "37"}])
def test_schedules_agree_bitwise(rr, tuning, env):
    """Every schedule of the fused fold (single pass, phased with and without
    barrier, compiled or run-time rank loop, both tile sizes, an odd grid)
    gives the same bits."""
    p, n = 8, 8 * (1 << 20) + 8 * 7 + 3
    x = W.random_inputs(65, p, n, "float32")
    want = C.all_reduce_fold(x, "sum", "float32")
    want_h = C.all_reduce_hier(x, "sum", "float32", 4)
    for k, v in env.items():
        tuning.set(k, v)
    assert_bitwise(run_ar(rr, x, "float32", "sum", "ring"), want, f"ring {env}")
    assert_bitwise(run_ar(rr, x, "float32", "sum", "hier", 4), want_h, f"hier {env}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("env", [{"RR_PHASE": "0"}, {}, {"RR_PHASE_SYNC": "0"}, {"RR_PHASE_STATIC": "0"},
                                 {"RR_PHASE_U": "4"}, {"RR_PHASE_GRID": "37"}, {"RR_PHASE_PER_CU": "8"},
                                 {"RR_PHASE_BATCH": "1"}, {"RR_PHASE_BATCH": "2"}, {"RR_PHASE_BATCH": "4"},
                                 {"RR_PHASE_BATCH": "4", "RR_PHASE_PER_CU": "1"},
                                 {"RR_PHASE_BATCH": "2", "RR_PHASE_STATIC": "0"}])
def test_reduce_scatter_and_reduce_schedules_agree(rr, tuning, env):
    """Reduce-scatter (one chunk per rank) and reduce (one output) through the
    single-pass kernel and every schedule of the phased one (with and without
    the batched rounds), at a size that takes several rounds: the same bits as
    the oracle."""
    p, L = 8, (1 << 20) + 8 * 3
    n = p * L
    x = W.random_inputs(66, p, n, "float32")
    want_rs = C.reduce_scatter_ring(x, "sum", "float32")
    want_red = C.reduce(x, "sum", "float32")
    for k, v in env.items():
        tuning.set(k, v)
    t0 = rr.barrier_timeouts()
    xs = to_dev(x, "float32")
    sh = torch.empty((p, L), dtype=torch.float32, device="cuda")
    rr.reduce_scatter(xs, sh)
    assert_bitwise(to_host(sh, "float32"), want_rs, f"reduce_scatter {env}")
    red = torch.empty(n, dtype=torch.float32, device="cuda")
    rr.reduce(xs, red, root=3)
    assert_bitwise(to_host(red, "float32"), want_red, f"reduce {env}")
    xb = W.random_inputs(67, p, n + 5, "bfloat16")  # a tail that is not a whole group
    red_b = torch.empty(n + 5, dtype=torch.bfloat16, device="cuda")
    rr.reduce(to_dev(xb, "bfloat16"), red_b)
    assert_bitwise(to_host(red_b, "bfloat16"), C.reduce(xb, "sum", "bfloat16"), f"reduce bf16 {env}")
    if env.get("RR_PHASE_PER_CU") != "8":
        assert rr.barrier_timeouts() == t0
    del xs, sh, red, red_b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("p,L,dtype", [(8, 24 << 18, "float32"), (8, (28 << 18) + 8 * 3 + 5, "float32"),
                                       (8, 10 << 20, "float32"), (8, (24 << 19) + 16, "bfloat16"), (5, 7 << 20, "int32")])
def test_reduce_scatter_and_reduce_partial_round(rr, p, L, dtype):
    """Reduce-scatter and reduce of 24-40 MiB per rank: one batched round that
    is at least 70% full, aligned and ragged chunks, p = 8 and 5."""
    n = p * L
    x = W.random_inputs(70, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    t0 = rr.barrier_timeouts()
    xs = to_dev(x, dtype)
    sh = torch.empty((p, L), dtype=xs.dtype, device="cuda")
    rr.reduce_scatter(xs, sh)
    assert_bitwise(to_host(sh, dtype), C.reduce_scatter_ring(x, "sum", dtype), f"reduce_scatter {p} {L} {dtype}")
    red = torch.empty(n, dtype=xs.dtype, device="cuda")
    rr.reduce(xs, red, root=1)
    assert_bitwise(to_host(red, dtype), C.reduce(x, "sum", dtype), f"reduce {p} {L} {dtype}")
    assert rr.barrier_timeouts() == t0
    del xs, sh, red
    torch.cuda.empty_cache()


@pytest.mark.parametrize("env", [{"RR_PHASE_BATCH": "2", "RR_PHASE_PER_CU": "1"},
                                 {"RR_PHASE_BATCH": "4", "RR_PHASE_PER_CU": "1"}])
@pytest.mark.parametrize("p,dtype,op", [(8, "float32", "sum"), (8, "float32", "max"), (8, "bfloat16", "sum"),
                                        (8, "float16", "avg"), (8, "int32", "min"), (5, "float32", "sum")])
def test_batched_rounds_ragged_chunks(rr, tuning, env, p, dtype, op):
    """The batched reduce-scatter and reduce where the chunk boundaries fall
    inside 16-byte groups (heads and tails, per-chunk tilings that differ),
    with one workgroup per CU so that 8 MiB per rank already takes several
    rounds: the same bits as the oracle."""
    L = (1 << 19) + 5
    n = p * L
    x = W.random_inputs(68, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    for k, v in env.items():
        tuning.set(k, v)
    t0 = rr.barrier_timeouts()
    xs = to_dev(x, dtype)
    sh = torch.empty((p, L), dtype=xs.dtype, device="cuda")
    rr.reduce_scatter(xs, sh, op=op)
    assert_bitwise(to_host(sh, dtype), C.reduce_scatter_ring(x, op, dtype), f"reduce_scatter {p} {dtype} {op} {env}")
    red = torch.empty(n, dtype=xs.dtype, device="cuda")
    rr.reduce(xs, red, root=p - 1, op=op)
    assert_bitwise(to_host(red, dtype), C.reduce(x, op, dtype), f"reduce {p} {dtype} {op} {env}")
    assert rr.barrier_timeouts() == t0
    del xs, sh, red
    torch.cuda.empty_cache()


AR_BATCH_CASES = [
    # (p, n, dtype, op): uniform chunks (interleaved runs), ragged chunks
    # (per-chunk tilings, heads and tails), 16-bit types, p = 5 (run-time
    # rank loop)
    (8, 8 << 20, "float32", "sum"),
    (8, (8 << 20) + 8 * 5 + 3, "float32", "max"),
    (8, 16 << 20, "bfloat16", "avg"),
    (8, (8 << 20) + 8 * 8 * 5, "float16", "sum"),
    (5, 5 * (3 << 21), "int32", "min"),
    # fewer tiles than one full round (16-44 MiB per rank): one partial round
    (8, 18 << 18, "float32", "sum"),
    (8, 7087872, "float32", "avg"),
    (8, (10 << 20) + 8 * 3 + 5, "bfloat16", "max"),
    (8, 10 << 20, "float32", "min"),
]


@pytest.mark.parametrize("env", [{}, {"RR_AR_BATCH": "2"}, {"RR_AR_BATCH": "4", "RR_PHASE_PER_CU": "1"},
                                 {"RR_AR_BATCH": "2", "RR_PHASE_STRIPS": "16"}, {"RR_PHASE_STRIPS": "8"},
                                 {"RR_PHASE_STRIPS": "64"},
                                 {"RR_AR_BATCH": "4", "RR_PHASE_STATIC": "0"}, {"RR_AR_BATCH": "1"}])
@pytest.mark.parametrize("case", range(len(AR_BATCH_CASES)))
def test_ring_all_reduce_batched_rounds(rr, tuning, env, case):
    """The ring all-reduce of several rounds in batched rounds (K tiles per
    workgroup and round, interleaved runs, the write phase output by output)
    and in single-tile rounds: the same bits as the oracle."""
    p, n, dtype, op = AR_BATCH_CASES[case]
    x = W.random_inputs(69 + case, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    want = C.all_reduce_fold(x, op, dtype)
    for k, v in env.items():
        tuning.set(k, v)
    t0 = rr.barrier_timeouts()
    assert_bitwise(run_ar(rr, x, dtype, op, "ring"), want, f"ring {p} {n} {dtype} {op} {env}")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


# Per-rank lengths whose one-round launch takes the tile of 4, 2 or 1 groups
# per lane (fewer 8-group tiles than CUs), with ragged chunk tails, p = 8
# (the kernels compiled for p = 8), 4 and 5 (the run-time loop).
SMALL = [(8, 1 << 20), (8, (1 << 19) + 13), (8, (1 << 18) + 3), (8, 65536), (8, 5000), (4, 1 << 19), (5, 300007),
         (8, (3 << 20) + 24)]


@pytest.mark.parametrize("p,n", SMALL)
@pytest.mark.parametrize("dtype", ("int32", "float32", "bfloat16", "float16"))
def test_small_one_round_tiles(rr, p, n, dtype):
    x = W.random_inputs(65, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    for op in ops:
        assert_bitwise(run_ar(rr, x, dtype, op, "ring"), C.all_reduce_ring(x, op, dtype), f"{op}")


# Per-rank lengths of one round with between one and two 8-group tiles per
# CU (the tile that spreads the launch most evenly: 2, 4 or 8 groups per
# lane, one tile per workgroup), aligned and ragged, p = 8 and 5.
SPREAD = [(8, 2228224, "float32"), (8, 2752512 + 8 * 7 + 3, "float32"), (8, 3538944, "float32"),
          (8, 4456448 + 8 * 3 + 5, "bfloat16"), (8, 5767168, "bfloat16"), (8, 7077888, "bfloat16"),
          (5, 5 * 530000 + 3, "float32"), (5, 5 * 1500000, "float16")]


@pytest.mark.parametrize("env", [{}, {"RR_AR_BATCH": "1"}])
@pytest.mark.parametrize("case", range(len(SPREAD)))
def test_one_round_spread_tiles(rr, tuning, env, case):
    """Between one and two tiles of 8 groups per lane per CU: the one-round
    tiles of 2, 4 or 8 groups, or above 1.5 per CU one batched round (with
    batches switched off, the 8-group round)."""
    p, n, dtype = SPREAD[case]
    x = W.random_inputs(67 + case, p, n, dtype, kind="normal")
    for k, v in env.items():
        tuning.set(k, v)
    for op in ("sum", "max", "avg"):
        assert_bitwise(run_ar(rr, x, dtype, op, "ring"), C.all_reduce_fold(x, op, dtype), f"{p} {n} {dtype} {op}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("p,n", [(8, 1 << 20), (8, (1 << 19) + 88), (8, 40000), (5, 300005), (8, (1 << 18) + 8)])
@pytest.mark.parametrize("dtype", ("int32", "float32", "bfloat16", "float16"))
def test_small_reduce_scatter_and_reduce_tiles(rr, p, n, dtype):
    """Reduce-scatter and reduce small enough for the tiles of 2 and 1
    groups per lane (chunks that are not whole 16-byte groups included)."""
    x = W.random_inputs(66, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    xs = to_dev(x, dtype)
    for op in ("sum", "min") + (("avg",) if dtype != "int32" else ()):
        outs = torch.empty((p, n // p), dtype=xs.dtype, device="cuda")
        rr.reduce_scatter(xs, outs, op=op)
        assert_bitwise(to_host(outs, dtype), C.reduce_scatter_ring(x, op, dtype), f"reduce_scatter {op}")
        if op == "avg":
            continue
        red = torch.empty(n, dtype=xs.dtype, device="cuda")
        rr.reduce(xs, red, root=0, op=op)
        assert_bitwise(to_host(red, dtype), C.reduce(x, op, dtype), f"reduce {op}")


# Interleaved tiles (runs of S tiles whose 256-group strips interleave) on
# uniform tilings with a partial last tile in every segment, in one round and
# in several: (collective, dtype, op, group, p, n).
STRIPED = [
    ("ring", "float32", "sum", 0, 8, 8 * 600012),
    ("ring", "int32", "max", 0, 8, 8 * 600012),
    ("ring", "bfloat16", "sum", 0, 8, 8 * 163864),
    ("ring", "float16", "sum", 0, 8, 8 * 163864),
    ("ring", "float32", "min", 0, 6, 6 * 900004),
    ("hier", "float32", "sum", 4, 8, 8 * 600012),
    ("hier", "bfloat16", "sum", 2, 8, 8 * 163864),
    ("reduce_scatter", "float32", "sum", 0, 8, 8 * 600012),
    ("reduce", "bfloat16", "sum", 0, 8, 8 * 600016),
]


@pytest.mark.parametrize("strips", ("0", "1", "3", "8"))
@pytest.mark.parametrize("coll,dtype,op,group,p,n", STRIPED)
def test_interleaved_tiles(rr, tuning, strips, coll, dtype, op, group, p, n):
    """Every tile layout of the phased fold (the schedule's default, forced
    contiguous, runs of 3 and of 8 interleaved tiles) gives the oracle's
    bits; no barrier waits out its bound."""
    kind = "full" if dtype == "int32" else ("fp16_patterns" if dtype == "float16" else "normal")
    x = W.random_inputs(69, p, n, dtype, kind=kind)
    tuning.set("RR_PHASE_STRIPS", strips)
    t0 = rr.barrier_timeouts()
    what = f"{coll} {dtype} {op} p={p} n={n} strips={strips}"
    if coll == "ring":
        assert_bitwise(run_ar(rr, x, dtype, op, "ring"), C.all_reduce_fold(x, op, dtype), what)
    elif coll == "hier":
        assert_bitwise(run_ar(rr, x, dtype, op, "hier", group), C.all_reduce_hier(x, op, dtype, group), what)
    elif coll == "reduce_scatter":
        xs = to_dev(x, dtype)
        sh = torch.empty((p, n // p), dtype=xs.dtype, device="cuda")
        rr.reduce_scatter(xs, sh, op=op)
        assert_bitwise(to_host(sh, dtype), C.reduce_scatter_ring(x, op, dtype), what)
    else:
        xs = to_dev(x, dtype)
        red = torch.empty(n, dtype=xs.dtype, device="cuda")
        rr.reduce(xs, red, op=op, root=2)
        assert_bitwise(to_host(red, dtype), C.reduce(x, op, dtype), what)
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()
