"""Pins of the CPU oracle to facts outside the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
a value printed on the pages, a closed form, a hand-derived IEEE-754 probe, a
library routine or brute force.  ``test_oracle.py`` runs them all;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle (on the
CPU) and checks that at least one pin catches each.

Pins resolve every oracle function through its module at call time, so a
monkeypatched mistake is seen.
"""

import json
import math
import os

import numpy as np

from oracle import bf16 as B
from oracle import collectives as C
from oracle import cost as K
from oracle import fp16 as H

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TWO24 = float(2 ** 24)


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def enc(values, dtype):
    """Python numbers (exactly representable) -> oracle storage array."""
    a = np.asarray(values, dtype=np.float64)
    if dtype == "int32":
        return a.astype(np.int32)
    if dtype == "float32":
        return a.astype(np.float32)
    if dtype == "float16":
        h = a.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), a), "test value not exactly representable in fp16"
        return h.view(np.uint16)
    f = a.astype(np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "test value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def dec(arr, dtype):
    """Oracle storage array -> float64 values (bf16 decoded by bit shifting and
    fp16 by numpy's float16 here, not by the oracle's codecs)."""
    arr = np.asarray(arr)
    if dtype == "float16":
        return np.ascontiguousarray(arr).view(np.float16).astype(np.float64)
    if dtype == "bfloat16":
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def bits(arr):
    arr = np.ascontiguousarray(arr)
    return arr.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[arr.itemsize])


# ---------------------------------------------------------------------------
# Worked example printed on page "分布式训练/推理", section "通信原语".

def pin_worked_example(dtype):
    g = _golden("worked_example.json")
    xs = enc(g["inputs"], dtype)
    p = g["p"]
    want = np.array(g["all_reduce"], dtype=np.float64)
    for f in (C.all_reduce_ring, C.all_reduce_fold):
        y = f(xs, "sum", dtype)
        assert y.shape == (p, 4)
        for r in range(p):
            assert np.array_equal(dec(y[r], dtype), want), (f.__name__, r, y[r])
    rs = C.reduce_scatter_ring(xs, "sum", dtype)
    assert np.array_equal(dec(rs, dtype), np.array(g["reduce_scatter"], dtype=np.float64)), rs
    ag = C.all_gather(rs)
    for r in range(p):
        assert np.array_equal(dec(ag[r], dtype), np.array(g["all_gather_of_reduce_scatter"], dtype=np.float64))
    # Reduce to one rank then broadcast has the same effect (page "LLM
    # Parallelism 基础", section "MPI Collective Operations").
    red = C.reduce(xs, "sum", dtype)
    assert np.array_equal(dec(red, dtype), want)
    bc = C.broadcast(red, p)
    assert np.array_equal(dec(bc, dtype), np.stack([want] * p))
    # The hierarchical variant reaches the same sum (2 groups of 2, 4 of 1, 1 of 4).
    for G in (1, 2, 4):
        h = C.all_reduce_hier(xs, "sum", dtype, G)
        assert np.array_equal(dec(h, dtype), np.stack([want] * p)), (G, h)


def pin_worked_example_max_min(dtype):
    """max/min of the same inputs, derived from the definitions: the largest
    input row is x_3 = [3,4,5,6], the smallest x_0 = [0,1,2,3]."""
    g = _golden("worked_example.json")
    xs = enc(g["inputs"], dtype)
    for op, want in (("max", [3, 4, 5, 6]), ("min", [0, 1, 2, 3])):
        for f in (C.all_reduce_ring, C.all_reduce_fold):
            y = f(xs, op, dtype)
            assert np.array_equal(dec(y, dtype), np.stack([np.array(want, float)] * 4)), (op, f.__name__)
        rs = C.reduce_scatter_ring(xs, op, dtype)
        assert np.array_equal(dec(rs, dtype).ravel(), np.array(want, float))
        assert np.array_equal(dec(C.reduce(xs, op, dtype), dtype), np.array(want, float))


# ---------------------------------------------------------------------------
# Closed form: x_r[j] = (j mod 16) + r  =>  sum y[j] = p (j mod 16) + p(p-1)/2,
# max y[j] = (j mod 16) + p - 1, min y[j] = j mod 16 (all exact in every dtype
# for the p used here).

def closed_form_inputs(p, n, dtype):
    j = np.arange(n) % 16
    return enc(np.stack([j + r for r in range(p)]), dtype)


def closed_form_expected(p, n, op):
    j = (np.arange(n) % 16).astype(np.float64)
    if op == "sum":
        return p * j + p * (p - 1) / 2
    if op == "max":
        return j + p - 1
    return j


def pin_closed_form(p, n, dtype):
    xs = closed_form_inputs(p, n, dtype)
    for op in C.OPS:
        want = closed_form_expected(p, n, op)
        for f in (C.all_reduce_ring, C.all_reduce_fold):
            y = f(xs, op, dtype)
            assert np.array_equal(dec(y, dtype), np.stack([want] * p)), (f.__name__, op, p, n)
        assert np.array_equal(dec(C.reduce(xs, op, dtype), dtype), want), (op, p, n)
        for G in [g for g in range(1, p + 1) if p % g == 0]:
            assert np.array_equal(dec(C.all_reduce_hier(xs, op, dtype, G), dtype), np.stack([want] * p))
        if n % p == 0:
            rs = C.reduce_scatter_ring(xs, op, dtype)
            L = n // p
            assert np.array_equal(dec(rs, dtype), want.reshape(p, L))
            assert np.array_equal(dec(C.all_gather(rs), dtype), np.stack([want] * p))


# ---------------------------------------------------------------------------
# Hand-derived IEEE-754 probes of the fold order.
#
# fp32 has a 24-bit significand: 2^24 + 1 is exactly halfway between 2^24 and
# 2^24 + 2 and rounds (ties to even) to 2^24, while -2^24 + 1 = -16777215 is
# exact.  So the order of the additions decides the result.

def ring_order_probe_inputs():
    """p = 4, n = 4, chunk c = element c.  Ring order folds chunk c as
    x_{c+1}, x_{c+2}, x_{c+3}, x_c; the probe puts 2^24, 1, 1, -2^24 there:
    (((2^24 + 1) + 1) - 2^24) = 0 in fp32.  Ascending rank order would give
    [2, 2, 2, 0]; starting at rank c, or running the ring backwards, gives
    [2, 2, 2, 2]."""
    p = 4
    rows = np.zeros((p, p), dtype=np.float64)
    for c in range(p):
        rows[(c + 1) % p, c] = TWO24
        rows[(c + 2) % p, c] = 1.0
        rows[(c + 3) % p, c] = 1.0
        rows[c % p, c] = -TWO24
    return rows


def pin_ring_order_probe(dtype):
    assert dtype in ("float32", "bfloat16")
    xs = enc(ring_order_probe_inputs(), dtype)
    want = np.zeros(4)
    for f in (C.all_reduce_ring, C.all_reduce_fold):
        y = f(xs, "sum", dtype)
        assert np.array_equal(dec(y, dtype), np.stack([want] * 4)), (f.__name__, y)
    rs = C.reduce_scatter_ring(xs, "sum", dtype)
    assert np.array_equal(dec(rs, dtype).ravel(), want), rs
    cols = xs
    got = C.fold_elements_ring_order(cols, np.arange(4), "sum", dtype)
    assert np.array_equal(dec(got, dtype), want), got


def pin_reduce_order_probe(dtype):
    """Reduce folds ranks 0..p-1: x = [2^24, 1, 1, -2^24] gives 0 in fp32
    (descending order would give 2)."""
    assert dtype in ("float32", "bfloat16")
    xs = enc(np.array([[TWO24], [1.0], [1.0], [-TWO24]]), dtype)
    assert dec(C.reduce(xs, "sum", dtype), dtype).tolist() == [0.0]


def hier_probe_inputs():
    """p = 8, groups of 4 = ranks {0..3} and {4..7}: x0 = 2^24, x2 = 1, x4 = 1,
    x5 = -2^24, the rest 0.  Group 0 folds to 2^24 (the 1 is lost), group 1 to
    1 - 2^24 = -16777215 (exact), and their sum is 1.  A flat fold in any rank
    order that meets 2^24 before both ones gives 0; groups taken by stride
    ({0,2,4,6}, {1,3,5,7}) give 0; rounding group 1's partial to bf16 at the
    representative gives -2^24 and then 0."""
    x = np.zeros((8, 1))
    x[0, 0] = TWO24
    x[2, 0] = 1.0
    x[4, 0] = 1.0
    x[5, 0] = -TWO24
    return x


def hier_probe_groups_of_2_inputs():
    """p = 8, groups of 2: partials g0 = 2^24, g1 = 1, g2 = 1, g3 = -2^24 fold
    ascending over groups to 0 (descending would give 2)."""
    x = np.zeros((8, 1))
    x[0, 0] = TWO24
    x[2, 0] = 1.0
    x[4, 0] = 1.0
    x[6, 0] = -TWO24
    return x


def pin_hier_probe(dtype):
    assert dtype in ("float32", "bfloat16")
    y = C.all_reduce_hier(enc(hier_probe_inputs(), dtype), "sum", dtype, 4)
    assert np.array_equal(dec(y, dtype), np.ones((8, 1))), y
    y2 = C.all_reduce_hier(enc(hier_probe_groups_of_2_inputs(), dtype), "sum", dtype, 2)
    assert np.array_equal(dec(y2, dtype), np.zeros((8, 1))), y2


# ---------------------------------------------------------------------------
# bf16 codec: round to nearest even, checked by hand and against torch (CPU).

def pin_bf16_rounding_hand():
    cases = [
        (1.0 + 2.0 ** -8, 0x3F80),          # halfway, even neighbour below
        (1.0 + 3 * 2.0 ** -8, 0x3F82),      # halfway, even neighbour above
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above halfway
        (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below halfway
        (TWO24 + 1.0, 0x4B80),              # fp32 rounds 2^24+1 first; bf16 of 2^24
        (-1.5, 0xBFC0),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float(np.finfo(np.float32).max), 0x7F80),  # rounds up to +inf
        (-float(np.finfo(np.float32).max), 0xFF80),
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
        (2.0 ** -133, 0x0001),              # smallest bf16 denormal (2^-126 * 2^-7)
        (2.0 ** -134, 0x0000),              # half of it: tie to even (0)
        (3 * 2.0 ** -134, 0x0002),          # 1.5 of it: tie to even (2)
    ]
    f = np.array([c[0] for c in cases], dtype=np.float32)
    got = B.narrow(f)
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    assert np.array_equal(got, want), [(hex(a), hex(b)) for a, b in zip(got, want)]
    # widen is exact: every bf16 pattern survives widen -> narrow unchanged
    # (non-NaN patterns) and widen places the 16 bits in the upper half.
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = B.widen(h)
    assert np.array_equal(w.view(np.uint32), h.astype(np.uint32) << 16)
    nonnan = (h & 0x7FFF) <= 0x7F80
    assert np.array_equal(B.narrow(w)[nonnan], h[nonnan])


def pin_bf16_nan():
    """A NaN keeps its sign and is quiet after narrowing, even when its payload
    sits only in the low 16 bits (truncation would turn it into an infinity)."""
    u = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0x7FA00000, 0xFFFFFFFF], dtype=np.uint32)
    got = B.narrow(u.view(np.float32))
    want = np.array([0x7FC0, 0xFFC0, 0x7FC0, 0x7FE0, 0xFFFF], dtype=np.uint16)
    assert np.array_equal(got, want), [hex(x) for x in got]


def pin_bf16_vs_torch(seed=7, count=1 << 20):
    """Independent check against torch's CPU float32 -> bfloat16 conversion
    (round to nearest even) on special classes and a stratified sample of bit
    patterns (NaNs excluded: torch returns one canonical NaN)."""
    import torch

    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2 ** 32, size=count, dtype=np.uint64).astype(np.uint32)
    # make sure every exponent and the tie / near-tie low halves are present
    u[: 1 << 16] = (np.arange(1 << 16, dtype=np.uint32) << 16) | np.uint32(0x8000)
    u[1 << 16: 2 << 16] = (np.arange(1 << 16, dtype=np.uint32) << 16) | np.uint32(0x7FFF)
    u[2 << 16: 3 << 16] = (np.arange(1 << 16, dtype=np.uint32) << 16) | np.uint32(0x8001)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(B.narrow(f), want)


def pin_bf16_ulp_distance(seed=5, count=1 << 16):
    """The bf16 ulp distance that the "at most 1 bf16 ulp" tolerance is read
    with: the number of steps between two values in the ordered list of all
    distinct non-NaN bf16 values (+0 and -0 one value, the infinities at the
    ends).  That list is built here by sorting every non-NaN pattern's value
    (decoded by bit shifting, not by the oracle's codec); hand cases pin the
    places where a sign-magnitude key goes wrong."""
    hand = [
        (0x3F80, 0x3F81, 1),  # 1 and its successor
        (0xBF80, 0xBF81, 1),  # the same below zero
        (0x0000, 0x8000, 0),  # +0 and -0 are one value
        (0x0001, 0x8001, 2),  # smallest denormals of both signs: -d, 0, +d
        (0x8000, 0x0001, 1),  # -0 to the smallest positive denormal
        (0x7F7F, 0x7F80, 1),  # largest finite to +inf
        (0xFF7F, 0xFF80, 1),  # most negative finite to -inf
        (0x7F80, 0xFF80, 2 * 0x7F80),  # -inf to +inf spans the whole list
        (0x4000, 0x3F80, 128),  # one binade of 7 mantissa bits: 1 -> 2
    ]
    a = np.array([h[0] for h in hand], dtype=np.uint16)
    b = np.array([h[1] for h in hand], dtype=np.uint16)
    want = np.array([h[2] for h in hand])
    got = B.ulp_distance(a, b)
    assert np.array_equal(got, want), list(zip(got.tolist(), want.tolist()))
    # brute force: rank of each value among the distinct non-NaN values
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    keep = (pats & 0x7FFF) <= 0x7F80
    vals = dec(pats[keep], "bfloat16")
    distinct = np.unique(vals)  # -0.0 == +0.0: one entry
    rank = dict(zip(pats[keep].tolist(), np.searchsorted(distinct, vals).tolist()))
    rng = np.random.default_rng(seed)
    pool = pats[keep]
    x = rng.choice(pool, size=count)
    y = rng.choice(pool, size=count)
    # neighbours too, where an off-by-one would show
    y[: count // 2] = np.clip(x[: count // 2].astype(np.int64) + rng.integers(-2, 3, size=count // 2), 0, 0xFFFF)
    y = y.astype(np.uint16)
    ok = (y & 0x7FFF) <= 0x7F80
    x, y = x[ok], y[ok]
    want = np.abs(np.array([rank[v] for v in x.tolist()]) - np.array([rank[v] for v in y.tolist()]))
    assert np.array_equal(B.ulp_distance(x, y), want)


# ---------------------------------------------------------------------------
# Integer and max/min rules.

def pin_int32_wrap():
    xs = np.array([[2 ** 31 - 1, -(2 ** 31), 5], [1, -1, -7]], dtype=np.int32)
    want = np.array([-(2 ** 31), 2 ** 31 - 1, -2], dtype=np.int32)
    for f in (C.all_reduce_ring, C.all_reduce_fold):
        assert np.array_equal(f(xs, "sum", "int32"), np.stack([want, want]))
    assert np.array_equal(C.reduce(xs, "sum", "int32"), want)


def pin_max_min_signed_zero():
    """p = 2, one element (chunk 1 holds it, so the fold is x_0 then x_1).
    Compare-and-select keeps the running value on ties: max(-0, +0) and
    min(-0, +0) with -0 first both give -0; with +0 first both give +0."""
    for first, second in ((-0.0, 0.0), (0.0, -0.0)):
        xs = np.array([[first], [second]], dtype=np.float32)
        for op in ("max", "min"):
            for f in (C.all_reduce_ring, C.all_reduce_fold):
                y = f(xs, op, "float32")
                assert np.all(np.signbit(y) == np.signbit(np.float32(first))), (op, first, y)
            red = C.reduce(xs, op, "float32")
            assert np.signbit(red[0]) == np.signbit(np.float32(first))
    # A chunk whose fold starts at rank 1: p = 2, n = 2, element 0 is chunk 0,
    # whose fold is x_1 then x_0.
    xs = np.array([[0.0, 0.0], [-0.0, 0.0]], dtype=np.float32)
    y = C.all_reduce_ring(xs, "max", "float32")
    assert np.signbit(y[0, 0]) and np.signbit(y[1, 0]), y


# ---------------------------------------------------------------------------
# Brute force on tiny random inputs.

def _wrap32(v):
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= (1 << 31) else v


def pin_bruteforce_int(seed):
    rng = np.random.default_rng(seed)
    for _ in range(25):
        p = int(rng.integers(1, 9))
        n = int(rng.integers(0, 65))
        big = bool(rng.integers(0, 2))
        lim = 2 ** 31 if big else 2 ** 20
        xs = rng.integers(-lim, lim, size=(p, n), dtype=np.int64).astype(np.int32)
        want_sum = np.array([_wrap32(sum(int(xs[r, j]) for r in range(p))) for j in range(n)], dtype=np.int32)
        want_max = np.array([max(int(xs[r, j]) for r in range(p)) for j in range(n)], dtype=np.int32)
        want_min = np.array([min(int(xs[r, j]) for r in range(p)) for j in range(n)], dtype=np.int32)
        for op, want in (("sum", want_sum), ("max", want_max), ("min", want_min)):
            for f in (C.all_reduce_ring, C.all_reduce_fold):
                assert np.array_equal(f(xs, op, "int32"), np.stack([want] * p)), (op, p, n)
            assert np.array_equal(C.reduce(xs, op, "int32"), want)
            if n % p == 0:
                assert np.array_equal(C.reduce_scatter_ring(xs, op, "int32").ravel(), want)
            for G in [g for g in range(1, p + 1) if p % g == 0]:
                assert np.array_equal(C.all_reduce_hier(xs, op, "int32", G), np.stack([want] * p))


def _gamma(k):
    u = 2.0 ** -24
    return k * u / (1 - k * u)


def pin_bruteforce_float(seed):
    """float32 sums lie within the a-priori bound of recursive summation,
    |y - exact| <= gamma_{p-1} * sum_r |x_r| (exact sum by math.fsum); bf16
    outputs add half an ulp of the result.  max/min equal numpy's reductions
    (no signed zeros or NaNs in these inputs).  Integer-valued float inputs
    give exact sums."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        p = int(rng.integers(1, 9))
        n = int(rng.integers(0, 65))
        x = rng.standard_normal((p, n)) * np.exp(rng.uniform(-8, 8, size=(p, n)))
        for dtype in ("float32", "bfloat16"):
            xs = enc(x.astype(np.float32).astype(np.float64), "float32") if dtype == "float32" else B.narrow(x.astype(np.float32))
            vals = dec(xs, dtype)
            exact = np.array([math.fsum(vals[:, j]) for j in range(n)])
            absum = np.abs(vals).sum(axis=0)
            outs = [C.all_reduce_ring(xs, "sum", dtype)[0], C.all_reduce_fold(xs, "sum", dtype)[0],
                    C.reduce(xs, "sum", dtype)]
            outs += [C.all_reduce_hier(xs, "sum", dtype, G)[0] for G in range(1, p + 1) if p % G == 0]
            for y in outs:
                err = np.abs(dec(y, dtype) - exact)
                bound = _gamma(max(p - 1, 0)) * absum * (1 + 1e-12)
                if dtype == "bfloat16":
                    bound = bound + np.abs(exact) * 2.0 ** -8 + 1e-300
                assert np.all(err <= bound), (dtype, p, n, err.max())
            for op, ref in (("max", np.max), ("min", np.min)):
                if n == 0:
                    continue
                want = ref(vals, axis=0)
                for y in (C.all_reduce_ring(xs, op, dtype)[0], C.all_reduce_fold(xs, op, dtype)[0],
                          C.reduce(xs, op, dtype)):
                    assert np.array_equal(dec(y, dtype), want), (op, dtype)
        ints = rng.integers(-1000, 1000, size=(p, n)).astype(np.float32)
        y = C.all_reduce_ring(ints, "sum", "float32")
        assert np.array_equal(y[0].astype(np.float64), ints.astype(np.float64).sum(axis=0))


# ---------------------------------------------------------------------------
# Identities and the schedule.

def random_inputs(rng, p, n, dtype):
    if dtype == "int32":
        return rng.integers(-(2 ** 31), 2 ** 31, size=(p, n), dtype=np.int64).astype(np.int32)
    f = rng.standard_normal((p, n)).astype(np.float32)
    return f if dtype == "float32" else B.narrow(f)


def pin_identities(seed):
    """all_reduce == all_gather(reduce_scatter) bitwise (page "分布式训练/推理",
    section "通信原语"); the schedule simulation equals the per-chunk formula
    bitwise; for int32 and max/min, all-reduce equals broadcast(reduce)
    (page "LLM Parallelism 基础", section "MPI Collective Operations")."""
    rng = np.random.default_rng(seed)
    for p in (1, 2, 3, 4, 8):
        for n in (0, p, 5 * p, 64 * p + p):
            for dtype in C.DTYPES:
                xs = random_inputs(rng, p, n, dtype)
                for op in C.OPS:
                    ar = C.all_reduce_ring(xs, op, dtype)
                    assert np.array_equal(bits(ar), bits(C.all_reduce_fold(xs, op, dtype)))
                    for r in range(p):
                        assert np.array_equal(bits(ar[r]), bits(ar[0]))
                    if n % p == 0:
                        ag = C.all_gather(C.reduce_scatter_ring(xs, op, dtype))
                        assert np.array_equal(bits(ag), bits(ar))
                    if dtype == "int32" or op != "sum":
                        bc = C.broadcast(C.reduce(xs, op, dtype), p)
                        assert np.array_equal(bits(bc), bits(ar)), (dtype, op)
                    chunk_of = np.searchsorted(np.array(C.chunk_bounds(n, p)[1:]), np.arange(n), side="right")
                    sampled = C.fold_elements_ring_order(xs, chunk_of, op, dtype)
                    assert np.array_equal(bits(sampled), bits(ar[0]))


def pin_schedule_symbolic(p):
    """Page "LLM Parallelism 基础", section "Ring AllReduce": 2(p-1) steps; in
    every step each rank sends exactly one chunk to the next rank and receives
    exactly one; after reduce-scatter rank c holds chunk c with every rank's
    contribution exactly once, gathered in the order c+1, c+2, ..., c; after
    all-gather every rank holds every chunk complete."""
    sched = C.ring_schedule(p)
    assert len(sched) == 2 * (p - 1) * p
    steps = sorted({(ph, s) for ph, s, *_ in sched})
    assert len(steps) == 2 * (p - 1)
    order = [[[r] for c in range(p)] for r in range(p)]  # order[rank][chunk]
    for ph, s in [("rs", s) for s in range(p - 1)] + [("ag", s) for s in range(p - 1)]:
        moves = [t for t in sched if t[0] == ph and t[1] == s]
        assert sorted(t[2] for t in moves) == list(range(p))
        assert sorted(t[3] for t in moves) == list(range(p))
        assert all(t[3] == (t[2] + 1) % p for t in moves)
        msgs = [list(order[t[2]][t[4]]) for t in moves]
        for (_, _, src, dst, c), msg in zip(moves, msgs):
            if ph == "rs":
                assert not set(msg) & set(order[dst][c])
                order[dst][c] = msg + order[dst][c]
            else:
                order[dst][c] = msg
        if ph == "rs" and s == p - 2:
            for c in range(p):
                assert order[c][c] == [(c + k) % p for k in range(1, p + 1)], (c, order[c][c])
    full = {c: [(c + k) % p for k in range(1, p + 1)] for c in range(p)}
    for r in range(p):
        for c in range(p):
            assert order[r][c] == full[c] or p == 1


def pin_hier_vs_flat(seed):
    """int32: hierarchical == flat bitwise; float32: within the recursive
    summation bound of each other."""
    rng = np.random.default_rng(seed)
    for p, G in ((8, 4), (8, 2), (6, 3), (4, 4), (4, 1)):
        xi = random_inputs(rng, p, 257, "int32")
        for op in C.OPS:
            assert np.array_equal(C.all_reduce_hier(xi, op, "int32", G), C.all_reduce_ring(xi, op, "int32"))
        xf = random_inputs(rng, p, 257, "float32")
        h = C.all_reduce_hier(xf, "sum", "float32", G)[0].astype(np.float64)
        f = C.all_reduce_ring(xf, "sum", "float32")[0].astype(np.float64)
        absum = np.abs(xf.astype(np.float64)).sum(axis=0)
        assert np.all(np.abs(h - f) <= 2 * _gamma(p - 1) * absum * (1 + 1e-12))
        for op in ("max", "min"):
            assert np.array_equal(C.all_reduce_hier(xf, op, "float32", G), C.all_reduce_ring(xf, op, "float32"))


def pin_edge_cases():
    for dtype in C.DTYPES:
        st = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16}[dtype]
        empty = np.zeros((4, 0), dtype=st)
        for op in C.OPS:
            assert C.all_reduce_ring(empty, op, dtype).shape == (4, 0)
            assert C.all_reduce_fold(empty, op, dtype).shape == (4, 0)
            assert C.reduce_scatter_ring(empty, op, dtype).shape == (4, 0)
            assert C.reduce(empty, op, dtype).shape == (0,)
        one = enc([[3, -2, 7]], dtype if dtype != "int32" else "int32")
        for op in C.OPS:
            assert np.array_equal(C.all_reduce_ring(one, op, dtype), one)
            assert np.array_equal(C.reduce(one, op, dtype), one[0])
        # fewer elements than ranks: some chunks are empty
        xs = enc([[1, 2], [3, 4], [5, 6], [7, 8], [9, 10]], dtype)
        y = C.all_reduce_ring(xs, "sum", dtype)
        assert np.array_equal(dec(y, dtype), np.stack([np.array([25.0, 30.0])] * 5))
    assert C.chunk_bounds(10, 4) == [0, 2, 5, 7, 10]
    assert C.chunk_bounds(2, 5) == [0, 0, 0, 1, 1, 2]


# ---------------------------------------------------------------------------
# binary16 codec: round to nearest even, by hand and against numpy's float16.

def pin_fp16_rounding_hand():
    cases = [
        (1.0 + 2.0 ** -11, 0x3C00),          # halfway, even neighbour below
        (1.0 + 3 * 2.0 ** -11, 0x3C02),      # halfway, even neighbour above
        (1.0 + 2.0 ** -11 + 2.0 ** -20, 0x3C01),  # just above halfway
        (65504.0, 0x7BFF),                   # largest finite
        (65519.0, 0x7BFF),                   # below the midpoint to 2^16
        (65520.0, 0x7C00),                   # the midpoint: ties to even = 2^16 = inf
        (-1.5, 0xBE00),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -14, 0x0400),                # smallest normal
        (2.0 ** -24, 0x0001),                # smallest subnormal
        (2.0 ** -25, 0x0000),                # half of it: tie to even (0)
        (3 * 2.0 ** -26, 0x0001),            # 0.75 of it rounds up
        (3 * 2.0 ** -25, 0x0002),            # 1.5 of it: tie to even (2)
        (2.0 ** -126, 0x0000),               # binary32 normal far below: 0
        (float("inf"), 0x7C00),
        (float("-inf"), 0xFC00),
    ]
    f = np.array([c[0] for c in cases], dtype=np.float32)
    got = H.narrow(f)
    want = np.array([c[1] for c in cases], dtype=np.uint16)
    assert np.array_equal(got, want), [(hex(a), hex(b)) for a, b in zip(got, want)]
    # NaNs stay NaN, keep the sign and are quiet
    u = np.array([0x7F800001, 0xFF800001, 0x7FC00000, 0x7FFFE000], dtype=np.uint32)
    nan = H.narrow(u.view(np.float32))
    assert np.array_equal(nan, np.array([0x7E00, 0xFE00, 0x7E00, 0x7FFF], dtype=np.uint16)), [hex(x) for x in nan]


def pin_fp16_vs_numpy(seed=11, count=1 << 20):
    """Against numpy's float16 conversions (an independent implementation of
    IEEE round to nearest even): every binary16 pattern widens to the value
    numpy gives it, and a stratified sample of binary32 patterns (every
    exponent with tie, near-tie and random low bits) narrows to numpy's
    pattern (NaNs excluded: numpy may keep other payload bits)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    w = H.widen(h)
    ref = h.view(np.float16).astype(np.float32)
    ok = ~np.isnan(ref)
    assert np.array_equal(w[ok].view(np.uint32), ref[ok].view(np.uint32))
    assert np.all(np.isnan(w[~ok]))
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 2 ** 32, size=count, dtype=np.uint64).astype(np.uint32)
    e = (np.arange(1 << 16, dtype=np.uint32) % 512) << 23
    u[: 1 << 16] = e | np.uint32(0x1000)       # tie at the normal-range rounding bit
    u[1 << 16: 2 << 16] = e | np.uint32(0x0FFF)
    u[2 << 16: 3 << 16] = e | (rng.integers(0, 1 << 23, size=1 << 16, dtype=np.uint64).astype(np.uint32))
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    with np.errstate(over="ignore"):
        ref16 = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(H.narrow(f), ref16)


def fp16_ring_order_probe_inputs():
    """The ring-order probe scaled by 2^-9 so that it fits binary16:
    2^15 + 2^-9 is halfway between two float32 neighbours (the float32 ulp
    at 2^15 is 2^-8) and rounds to 2^15, so ring order gives 0 while the
    ascending fold gives [2^-8, 2^-8, 2^-8, 0]."""
    return ring_order_probe_inputs() * 2.0 ** -9


def pin_fp16_order_probes():
    xs = enc(fp16_ring_order_probe_inputs(), "float16")
    for f in (C.all_reduce_ring, C.all_reduce_fold):
        assert np.array_equal(dec(f(xs, "sum", "float16"), "float16"), np.zeros((4, 4))), f.__name__
    assert np.array_equal(dec(C.reduce(xs, "sum", "float16"), "float16"), np.array([2.0 ** -8] * 3 + [0.0]))
    hx = enc(hier_probe_inputs() * 2.0 ** -9, "float16")
    assert np.array_equal(dec(C.all_reduce_hier(hx, "sum", "float16", 4), "float16"), np.full((8, 1), 2.0 ** -9))
    for op, want in (("sum", [6, 10, 14, 18]), ("max", [3, 4, 5, 6]), ("min", [0, 1, 2, 3])):
        g = _golden("worked_example.json")
        y = C.all_reduce_fold(enc(g["inputs"], "float16"), op, "float16")
        assert np.array_equal(dec(y, "float16"), np.stack([np.array(want, float)] * 4)), op


def pin_fp16_sum_rounds_once():
    """Sixteen-bit inputs are folded in float32 and rounded once: p = 3,
    x = [1, 2^-11, 2^-11] sums to 1 + 2^-10 exactly in float32, which is a
    binary16 value; rounding each partial to binary16 would lose both
    halves (1 + 2^-11 ties to 1)."""
    xs = enc([[1.0], [2.0 ** -11], [2.0 ** -11]], "float16")
    for y in (C.all_reduce_fold(xs, "sum", "float16")[0], C.reduce(xs, "sum", "float16")):
        assert dec(y, "float16").tolist() == [1.0 + 2.0 ** -10]


# ---------------------------------------------------------------------------
# AVG: the averaged gradient g = (1/p) sum_r grad_r of page "分布式训练/推理"
# (data parallelism), read as the op's sum fold, one division by p, one
# conversion.

def pin_avg_worked_example():
    """The worked example's all-reduce [6, 10, 14, 18] over p = 4 ranks
    averages to [1.5, 2.5, 3.5, 4.5] (exact in every float dtype)."""
    g = _golden("worked_example.json")
    want = np.array([1.5, 2.5, 3.5, 4.5])
    for dtype in ("float32", "bfloat16", "float16"):
        xs = enc(g["inputs"], dtype)
        for f in (C.all_reduce_ring, C.all_reduce_fold):
            assert np.array_equal(dec(f(xs, "avg", dtype), dtype), np.stack([want] * 4)), (dtype, f.__name__)
        assert np.array_equal(dec(C.reduce_scatter_ring(xs, "avg", dtype), dtype).ravel(), want), dtype
        assert np.array_equal(dec(C.reduce(xs, "avg", dtype), dtype), want), dtype
        for G in (1, 2, 4):
            assert np.array_equal(dec(C.all_reduce_hier(xs, "avg", dtype, G), dtype), np.stack([want] * 4))


def pin_avg_closed_form(p, n):
    """x_r[j] = (j mod 16) + r averages to (j mod 16) + (p - 1)/2: the sum is
    exact and so is its quotient by p, which IEEE division returns unchanged."""
    j = (np.arange(n) % 16).astype(np.float64)
    want = j + (p - 1) / 2.0
    for dtype in ("float32", "bfloat16", "float16"):
        xs = closed_form_inputs(p, n, dtype) if dtype != "float16" else enc(np.stack([j + r for r in range(p)]), dtype)
        for f in (C.all_reduce_ring, C.all_reduce_fold):
            assert np.array_equal(dec(f(xs, "avg", dtype), dtype), np.stack([want] * p)), (dtype, p, n)
        assert np.array_equal(dec(C.reduce(xs, "avg", dtype), dtype), want)


def pin_avg_division_probes():
    """Hand-derived float32 probes of how the mean is formed (p = 3):
    * x = [1, 2, 2]: the division 5/3 rounds to 0x3FD55555; multiplying by a
      rounded 1/3 (0x3EAAAAAB) gives 0x3FD55556 instead.
    * x = [2, 1, 4]: dividing the sum, fl(7/3) = 0x40155555; dividing each
      term first gives 2/3 + 1/3 + 4/3 = 0x40155556.
    * bf16 x = [1, 1.5, 2^-7]: the float32 sum 2.5078125 divided by 3 is
      exactly 0.8359375 = bf16 0x3F56; rounding the sum to bf16 before the
      division (2.5, a tie to even) gives 0.83203125 = 0x3F55."""
    xs = np.array([[1.0], [2.0], [2.0]], dtype=np.float32)
    for y in (C.all_reduce_fold(xs, "avg", "float32")[0], C.reduce(xs, "avg", "float32"),
              C.all_reduce_ring(xs, "avg", "float32")[0]):
        assert int(y.view(np.uint32)[0]) == 0x3FD55555, hex(int(y.view(np.uint32)[0]))
    xs = np.array([[2.0], [1.0], [4.0]], dtype=np.float32)
    for y in (C.all_reduce_fold(xs, "avg", "float32")[0], C.reduce(xs, "avg", "float32")):
        assert int(y.view(np.uint32)[0]) == 0x40155555, hex(int(y.view(np.uint32)[0]))
    xb = enc([[1.0], [1.5], [2.0 ** -7]], "bfloat16")
    for y in (C.all_reduce_fold(xb, "avg", "bfloat16")[0], C.reduce(xb, "avg", "bfloat16"),
              C.all_reduce_hier(xb, "avg", "bfloat16", 3)[0]):
        assert int(y[0]) == 0x3F56, hex(int(y[0]))


def pin_avg_correctly_rounded(seed):
    """The float32 mean is the correctly rounded quotient of the float32 sum
    (the sum itself is pinned elsewhere): computed here in binary64 and
    rounded to binary32, which for a quotient of two binary32 values is
    correctly rounded because 53 >= 2*24 + 2 (Figueroa, "When is double
    rounding innocuous?", 1995).  The ring's sum is taken from the sum op."""
    rng = np.random.default_rng(seed)
    for p in (2, 3, 5, 6, 7, 8):
        xs = (rng.standard_normal((p, 97)) * np.exp(rng.uniform(-20, 20, size=(p, 97)))).astype(np.float32)
        s = C.all_reduce_fold(xs, "sum", "float32")[0]
        want = (s.astype(np.float64) / p).astype(np.float32)
        got = C.all_reduce_fold(xs, "avg", "float32")[0]
        assert np.array_equal(bits(got), bits(want)), p
        rs = C.reduce_scatter_ring(xs[:, : (97 // p) * p], "avg", "float32").ravel()
        s2 = C.all_reduce_fold(xs[:, : (97 // p) * p], "sum", "float32")[0]
        assert np.array_equal(bits(rs), bits((s2.astype(np.float64) / p).astype(np.float32)))
        r = C.reduce(xs, "avg", "float32")
        assert np.array_equal(bits(r), bits((C.reduce(xs, "sum", "float32").astype(np.float64) / p).astype(np.float32)))


def pin_avg_ring_order_and_int():
    """AVG keeps the ring's fold order (the ring probe averages to 0, not to
    the ascending fold's 0.5), and is refused for int32."""
    xs = enc(ring_order_probe_inputs(), "float32")
    assert np.array_equal(C.all_reduce_ring(xs, "avg", "float32"), np.zeros((4, 4), np.float32))
    assert np.array_equal(C.all_reduce_fold(xs, "avg", "float32"), np.zeros((4, 4), np.float32))
    for fn in (lambda: C.all_reduce_fold(np.ones((2, 2), np.int32), "avg", "int32"),
               lambda: C.reduce(np.ones((2, 2), np.int32), "avg", "int32")):
        try:
            fn()
        except ValueError:
            continue
        raise AssertionError("avg over int32 was accepted")


# ---------------------------------------------------------------------------
# Scatter and gather (page "分布式训练/推理", section "通信原语"; page "LLM
# Parallelism 基础", table of MPI collectives: rank 0 cuts the array into p
# pieces, one per process; gather collects every process's piece at one).

def pin_scatter_gather():
    g = _golden("worked_example.json")
    # the reduce-scatter of the worked example is the scatter of its all-reduce
    for dtype in ("int32", "float32", "bfloat16", "float16"):
        ar = C.all_reduce_fold(enc(g["inputs"], dtype), "sum", dtype)[0]
        sc = C.scatter(ar, 4)
        assert np.array_equal(dec(sc, dtype), np.array(g["reduce_scatter"], dtype=np.float64))
        assert np.array_equal(dec(C.gather(sc), dtype), np.array(g["all_gather_of_reduce_scatter"], float))
    rng = np.random.default_rng(5)
    for p in (1, 2, 3, 8):
        for L in (0, 1, 7):
            x = rng.integers(-100, 100, size=p * L).astype(np.int32)
            sc = C.scatter(x, p)
            assert sc.shape == (p, L)
            for c in range(p):
                for j in range(L):
                    assert sc[c, j] == x[c * L + j]
            assert np.array_equal(C.gather(sc), x)
            # reduce-scatter is the scatter of the reduced vector (order-free ops)
            xs = rng.integers(-(2 ** 31), 2 ** 31, size=(p, p * L), dtype=np.int64).astype(np.int32)
            for op in C.OPS:
                assert np.array_equal(C.reduce_scatter_ring(xs, op, "int32"), C.scatter(C.reduce(xs, op, "int32"), p))
            # the gathered reduce-scatter is the ring all-reduce (float32, bitwise)
            xf = rng.standard_normal((p, p * L)).astype(np.float32)
            rs = C.reduce_scatter_ring(xf, "sum", "float32")
            assert np.array_equal(bits(C.gather(rs)), bits(C.all_reduce_fold(xf, "sum", "float32")[0]))
    try:
        C.scatter(np.zeros(5, np.int32), 2)
    except ValueError:
        pass
    else:
        raise AssertionError("scatter of 5 elements over 2 ranks was accepted")


# ---------------------------------------------------------------------------
# Bucketed all-reduce: the tensors of a bucket are laid end to end and the
# ring chunks the bucket, not each tensor.

def pin_bucket():
    """The ring probe cut into tensors of 1 and 3 elements still folds each
    element in its bucket chunk's ring order (all zeros); chunking each
    tensor on its own would put the 1-element tensor's element in chunk 3 of
    its own ring (order x_0, x_1, x_2, x_3) and give 2.  A one-tensor bucket
    is the plain all-reduce; integer buckets equal the per-element sum; the
    worked example and the closed form hold across tensor cuts."""
    xs = enc(ring_order_probe_inputs(), "float32")
    for cut in ((1, 3), (2, 2), (3, 1), (1, 1, 1, 1)):
        parts, o = [], 0
        for w in cut:
            parts.append(np.ascontiguousarray(xs[:, o:o + w]))
            o += w
        for dtype in ("float32",):
            out = C.all_reduce_bucket(parts, "sum", dtype)
            assert [t.shape for t in out] == [t.shape for t in parts]
            for t in out:
                assert np.array_equal(t, np.zeros_like(t)), (cut, out)
    rng = np.random.default_rng(9)
    for p in (1, 3, 8):
        sizes = [int(v) for v in rng.integers(0, 40, size=5)]
        ts = [rng.integers(-(2 ** 31), 2 ** 31, size=(p, m), dtype=np.int64).astype(np.int32) for m in sizes]
        for op in C.OPS:
            out = C.all_reduce_bucket(ts, op, "int32")
            for t, y in zip(ts, out):
                want = C.reduce(t, op, "int32")
                assert np.array_equal(y, np.stack([want] * p)), (p, op)
        xf = rng.standard_normal((p, 50)).astype(np.float32)
        one = C.all_reduce_bucket([xf], "sum", "float32")[0]
        assert np.array_equal(bits(one), bits(C.all_reduce_fold(xf, "sum", "float32")))
    g = _golden("worked_example.json")
    for dtype in ("float32", "bfloat16", "float16"):
        x = enc(g["inputs"], dtype)
        out = C.all_reduce_bucket([x[:, :1], x[:, 1:]], "avg", dtype)
        assert np.array_equal(dec(np.concatenate(out, axis=1), dtype), np.stack([np.array([1.5, 2.5, 3.5, 4.5])] * 4))
    p, n = 8, 4099
    xs = closed_form_inputs(p, n, "float32")
    out = C.all_reduce_bucket([xs[:, :1000], xs[:, 1000:1001], xs[:, 1001:]], "sum", "float32")
    assert np.array_equal(dec(np.concatenate(out, axis=1), "float32"), np.stack([closed_form_expected(p, n, "sum")] * p))


# ---------------------------------------------------------------------------
# Tensor-parallel layouts (page "分布式训练/推理", tensor parallelism: the
# all-gather of [B, d/p] outputs concatenated along dim 1, and the scatter
# strategy, whose partial [B, D] outputs are summed and cut into feature
# slices).

def pin_all_gather_dim1():
    rng = np.random.default_rng(3)
    for p, B_, w in ((1, 3, 2), (2, 1, 1), (4, 3, 5), (8, 2, 3)):
        sh = rng.integers(-50, 50, size=(p, B_, w)).astype(np.int32)
        y = C.all_gather_dim1(sh)
        assert y.shape == (p, B_, p * w)
        for r in range(p):
            for b in range(B_):
                for c in range(p):
                    for j in range(w):
                        assert y[r, b, c * w + j] == sh[c, b, j]
        # the column slices of a matrix gather back into the matrix
        M = rng.standard_normal((B_, p * w)).astype(np.float32)
        cols = np.stack([M[:, c * w:(c + 1) * w] for c in range(p)])
        assert np.array_equal(C.all_gather_dim1(cols)[p - 1], M)


def pin_reduce_scatter_cols():
    """Row-parallel partial outputs: H_r W_r summed over r is H W (exact for
    small integers), and rank c keeps feature slice c.  The fold order of
    slice c is the ring order of chunk c: the ring probe laid out as a
    1 x 4 row (and as two rows) gives zeros."""
    rng = np.random.default_rng(4)
    for p, B_, K, D in ((2, 3, 4, 6), (4, 2, 8, 8), (8, 5, 16, 24)):
        H_ = rng.integers(-8, 8, size=(B_, K)).astype(np.float64)
        W_ = rng.integers(-8, 8, size=(K, D)).astype(np.float64)
        k = K // p
        parts = np.stack([H_[:, r * k:(r + 1) * k] @ W_[r * k:(r + 1) * k, :] for r in range(p)]).astype(np.float32)
        full = H_ @ W_
        got = C.reduce_scatter_cols(parts, "sum", "float32")
        w = D // p
        assert got.shape == (p, B_, w)
        for c in range(p):
            assert np.array_equal(got[c].astype(np.float64), full[:, c * w:(c + 1) * w]), (p, c)
        pi = parts.astype(np.int32)
        for op in C.OPS:
            red = C.reduce(pi.reshape(p, B_ * D), op, "int32").reshape(B_, D)
            got = C.reduce_scatter_cols(pi, op, "int32")
            for c in range(p):
                assert np.array_equal(got[c], red[:, c * w:(c + 1) * w])
    probe = ring_order_probe_inputs().astype(np.float32)
    for rows in (probe[:, None, :], np.stack([probe, probe], axis=1)):
        got = C.reduce_scatter_cols(rows, "sum", "float32")
        assert np.array_equal(got, np.zeros_like(got)), got
    # an all-gather along dim 1 of the slices gives every rank the summed matrix
    xs = rng.standard_normal((4, 3, 8)).astype(np.float32)
    ag = C.all_gather_dim1(C.reduce_scatter_cols(xs, "sum", "float32"))
    flat = C.all_reduce_fold(np.ascontiguousarray(xs.transpose(0, 2, 1)).reshape(4, 24), "sum", "float32")[0]
    assert np.array_equal(bits(ag[0]), bits(np.ascontiguousarray(flat.reshape(8, 3).T)))


# ---------------------------------------------------------------------------
# Hierarchical variants (page "大模型并行的最小闭环", "Source Log: 2026-05-05").

def pin_hier_variants():
    """intra="ring": with one group the hierarchical all-reduce is the ring
    all-reduce of the group (the ring probe gives zeros, the ascending
    default [2, 2, 2, 0]); integer results and exact sums do not depend on
    the variant.  wire_round: p = 4, G = 2, bf16 x = [1, 2^-8, 2^-8, 0]; the
    group partial 1 + 2^-8 rounds (tie to even) to 1 on the wire and the
    result is 1 (the next tie), while float32 partials give 1 + 2^-7."""
    xs = enc(ring_order_probe_inputs(), "float32")
    assert np.array_equal(C.all_reduce_hier(xs, "sum", "float32", 4, intra="ring"), np.zeros((4, 4), np.float32))
    assert np.array_equal(C.all_reduce_hier(xs, "sum", "float32", 4)[0], np.array([2, 2, 2, 0], np.float32))
    # two groups of 4, each a copy of the probe, scaled: group partials from the
    # ring are 0, so the result is 0 (the ascending intra fold gives 2*[2,2,2,0])
    x8 = np.concatenate([xs, xs])
    assert np.array_equal(C.all_reduce_hier(x8, "sum", "float32", 4, intra="ring"), np.zeros((8, 4), np.float32))
    rng = np.random.default_rng(6)
    for p, G in ((8, 4), (8, 2), (6, 3), (4, 4)):
        xi = rng.integers(-(2 ** 31), 2 ** 31, size=(p, 37), dtype=np.int64).astype(np.int32)
        for op in C.OPS:
            for kw in ({"intra": "ring"}, {"wire_round": True}, {"intra": "ring", "wire_round": True}):
                assert np.array_equal(C.all_reduce_hier(xi, op, "int32", G, **kw), C.all_reduce_fold(xi, op, "int32"))
        xc = closed_form_inputs(p, 100, "bfloat16")
        for kw in ({"intra": "ring"}, {"wire_round": True}):
            assert np.array_equal(dec(C.all_reduce_hier(xc, "sum", "bfloat16", G, **kw), "bfloat16"),
                                  np.stack([closed_form_expected(p, 100, "sum")] * p))
        xf = rng.standard_normal((p, 37)).astype(np.float32)
        assert np.array_equal(C.all_reduce_hier(xf, "sum", "float32", G, wire_round=True),
                              C.all_reduce_hier(xf, "sum", "float32", G))
    xb = enc([[1.0], [2.0 ** -8], [2.0 ** -8], [0.0]], "bfloat16")
    assert dec(C.all_reduce_hier(xb, "sum", "bfloat16", 2, wire_round=True), "bfloat16")[:, 0].tolist() == [1.0] * 4
    assert dec(C.all_reduce_hier(xb, "sum", "bfloat16", 2), "bfloat16")[:, 0].tolist() == [1.0 + 2.0 ** -7] * 4


# ---------------------------------------------------------------------------
# Alpha-beta cost model.

def pin_cost_ring():
    """With no latency, bandwidth times the ring's time is what one rank sends
    in the schedule (counted from the oracle's own transfer list); with no
    bytes it is alpha times the schedule's number of steps; p = 1 costs
    nothing."""
    for p in (2, 3, 4, 8, 16):
        n = p * 1000
        sched = C.ring_schedule(p)
        b = C.chunk_bounds(n, p)
        sent = sum(b[c + 1] - b[c] for (_, _, src, _, c) in sched if src == 0) * 4.0
        t = K.ring_all_reduce(p, n * 4.0, 0.0, 1.0)
        assert abs(t - sent) <= 1e-9 * sent, (p, t, sent)
        steps = len({(ph, st) for ph, st, *_ in sched})
        assert abs(K.ring_all_reduce(p, 0.0, 1e-6, 1e9) - steps * 1e-6) <= 1e-12 * steps * 1e-6
    assert K.ring_all_reduce(1, 1e6, 1e-6, 1e9) == 0.0


def pin_cost_hier_example():
    """Page "大模型并行的最小闭环", section "Source Log: 2026-05-05": 2 nodes of
    4 GPUs holding B = 8 MB each.  Without the hierarchy a node ships
    4 x 8 MB = 32 MB across nodes, with it 8 MB: four times less (= N).  With
    the link speeds of the table on page "分布式训练/推理" (NVLink about 1.8
    TB/s, InfiniBand about 0.05 TB/s) and no latency: flat 32e6/0.05e12 =
    640 us; hierarchical 32e6/1.8e12 + 8e6/0.05e12 = 17.78 + 160 = 177.78 us."""
    B_, N = 8e6, 4
    nv, ib = (0.0, 1.8e12), (0.0, 0.05e12)
    t_flat, t_hier = K.hier_all_reduce(N, B_, nv, ib)
    assert abs(t_flat - 640e-6) < 1e-12
    assert abs(t_hier - (32e6 / 1.8e12 + 160e-6)) < 1e-12
    assert abs(t_flat * ib[1] - 32e6) < 1e-3  # bytes a node ships without the hierarchy
    # with the intra-node step free, the hierarchy is exactly N times faster
    tf, th = K.hier_all_reduce(N, B_, (0.0, 1e300), ib)
    assert abs(tf / th - N) < 1e-9
    # a latency-bound case: tiny messages, where the extra fast step costs more than it saves
    tf, th = K.hier_all_reduce(N, 8.0, (5e-6, 1.8e12), (1e-6, 0.05e12))
    assert th > tf
