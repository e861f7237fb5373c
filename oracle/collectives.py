"""Plain, slow, obviously-correct collective reductions (test infrastructure).

Every function takes the p rank buffers as a 2-D NumPy array ``xs`` of shape
(p, n): row r is rank r's buffer.  Storage types:

    "int32"    -> numpy.int32
    "float32"  -> numpy.float32
    "bfloat16" -> numpy.uint16 holding bf16 bit patterns (see ``bf16``)
    "float16"  -> numpy.uint16 holding IEEE binary16 bit patterns (see ``fp16``)

Accumulator type (the type every partial result is held in): int32 for int32,
float32 for float32, bfloat16 and float16 (16-bit inputs are widened exactly,
folded in float32 and rounded to their storage type once, at the end).

Readings of what the pages leave open (each one is also listed in the design
notes of the repository):

* Ring direction: every rank sends to rank r+1 (mod p) -- "the next card on
  the ring" in page "LLM Parallelism 基础", section "Ring AllReduce".
* Which chunk moves at which step: in reduce-scatter step s (0-based) rank r
  sends chunk (r-1-s) mod p; in all-gather step s it sends chunk (r-s) mod p.
  It is the only assignment with that direction that leaves rank c holding
  the reduced chunk c after p-1 steps, which the same section states (and
  which the worked example of page "分布式训练/推理", section "通信原语",
  shows: rank 0 receives [6]).
* The receiver combines ``op(message, local)``: the partial that arrives is
  the running accumulator, the local value is the next term.  For chunk c the
  fold order is therefore x_{c+1}, x_{c+2}, ..., x_{c+p-1}, x_c (mod p).
* Uneven split: the pages cut the data evenly.  When p does not divide n the
  chunk bounds are floor(c*n/p); reduce-scatter and all-gather require p | n.
* Reduce folds ranks in ascending order 0..p-1, the order of the sum in the
  all-reduce formula of page "分布式训练/推理"; the pages give no reduce
  algorithm.
* Sum of int32 wraps modulo 2**32 (two's complement).
* max / min are compare-and-select with the running value as first operand:
  max keeps the running value unless the new value is strictly greater (min:
  strictly less).  Ties, including +0 against -0, keep the earlier operand;
  a NaN running value stays; a NaN new value is skipped.
* Hierarchical: contiguous groups [jG, jG+G), representative = the group's
  first rank; group partials fold ascending in the accumulator type and stay
  in it (no rounding at the representative); the representatives' partials
  fold ascending over groups; one final conversion; every rank receives the
  result.
* AVG (page "分布式训练/推理": the DDP gradient g = (1/p) sum_r grad L_r, and the
  sharded optimizer's fallback "SUM, then /= world_size"): the sum fold in the
  op's order, then one IEEE division of the accumulator by p, then the one
  conversion to storage.  Defined for floating-point dtypes only.
"""

import numpy as np

from . import bf16, fp16

DTYPES = ("int32", "float32", "bfloat16")
OPS = ("sum", "max", "min")
ALL_DTYPES = DTYPES + ("float16",)
ALL_OPS = OPS + ("avg",)

_STORAGE = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16, "float16": np.uint16}


def _check(xs, dtype, op=None):
    if dtype not in _STORAGE:
        raise ValueError(f"unknown dtype {dtype!r}")
    if op is not None and op not in ALL_OPS:
        raise ValueError(f"unknown op {op!r}")
    if op == "avg" and dtype == "int32":
        raise ValueError("avg is defined for floating-point dtypes only")
    xs = np.asarray(xs)
    if xs.ndim != 2:
        raise ValueError("xs must have shape (p, n)")
    if xs.dtype != _STORAGE[dtype]:
        raise TypeError(f"{dtype} buffers must be stored as {_STORAGE[dtype].__name__}")
    return xs


def to_acc(x, dtype):
    """One rank's buffer (or a slice of it) -> a fresh accumulator-type copy."""
    if dtype == "bfloat16":
        return bf16.widen(x)
    if dtype == "float16":
        return fp16.widen(x)
    return np.array(x, dtype=_STORAGE[dtype], copy=True)


def from_acc(a, dtype):
    """Accumulator values -> storage type (one rounding, for 16-bit types only)."""
    if dtype == "bfloat16":
        return bf16.narrow(a)
    if dtype == "float16":
        return fp16.narrow(a)
    return np.array(a, dtype=_STORAGE[dtype], copy=True)


def combine(acc, v, op):
    """One fold step: the running value ``acc`` combined with the next term ``v``."""
    if op in ("sum", "avg"):
        return acc + v  # NumPy array addition: IEEE RNE for float32, wrap for int32
    if op == "max":
        return np.where(v > acc, v, acc)
    if op == "min":
        return np.where(v < acc, v, acc)
    raise ValueError(f"unknown op {op!r}")


def finish(acc, op, p):
    """After the fold: AVG divides the accumulator by p (one IEEE division,
    round to nearest even, in float32); every other op leaves it unchanged."""
    if op == "avg":
        return acc / np.float32(p)
    return acc


def chunk_bounds(n, p):
    """Start of every chunk plus the end: [floor(c*n/p) for c in 0..p]."""
    return [(c * n) // p for c in range(p + 1)]


def ring_schedule(p):
    """The ring's transfers as (phase, step, src, dst, chunk) tuples.

    Page "LLM Parallelism 基础", section "Ring AllReduce": phase "rs" has p-1
    steps in which each rank passes one chunk to the next rank and the
    receiver accumulates; phase "ag" has p-1 steps in which the receiver
    overwrites.  2(p-1) steps, p transfers per step.
    """
    out = []
    for s in range(p - 1):
        for r in range(p):
            out.append(("rs", s, r, (r + 1) % p, (r - 1 - s) % p))
    for s in range(p - 1):
        for r in range(p):
            out.append(("ag", s, r, (r + 1) % p, (r - s) % p))
    return out


def simulate_ring(xs, op, dtype, phases=("rs", "ag")):
    """Run the ring schedule literally on p separate accumulator buffers.

    Returns the list of p buffers (accumulator type) after the given phases.
    Within one step every message is read before any receiver updates (all
    ranks send at once).
    """
    xs = _check(xs, dtype, op)
    p, n = xs.shape
    b = chunk_bounds(n, p)
    buf = [to_acc(xs[r], dtype) for r in range(p)]
    sched = ring_schedule(p)
    for phase in phases:
        if phase == "ag":
            # the owner of each reduced chunk applies the op's final step (AVG:
            # the division by p) before the chunk travels round the ring
            for c in range(p):
                buf[c][b[c]:b[c + 1]] = finish(buf[c][b[c]:b[c + 1]], op, p)
        for s in range(p - 1):
            moves = [t for t in sched if t[0] == phase and t[1] == s]
            msgs = [buf[src][b[c]:b[c + 1]].copy() for (_, _, src, _, c) in moves]
            for (_, _, _, dst, c), msg in zip(moves, msgs):
                lo, hi = b[c], b[c + 1]
                if phase == "rs":
                    buf[dst][lo:hi] = combine(msg, buf[dst][lo:hi], op)
                else:
                    buf[dst][lo:hi] = msg
    return buf


def all_reduce_ring(xs, op, dtype):
    """Ring all-reduce (reduce-scatter then all-gather); shape (p, n) result."""
    buf = simulate_ring(xs, op, dtype)
    return np.stack([from_acc(bb, dtype) for bb in buf])


def reduce_scatter_ring(xs, op, dtype):
    """Ring reduce-scatter: row c of the (p, n/p) result is reduced chunk c."""
    xs = _check(xs, dtype, op)
    p, n = xs.shape
    if n % p:
        raise ValueError("reduce-scatter needs p | n")
    buf = simulate_ring(xs, op, dtype, phases=("rs",))
    L = n // p
    return np.stack([from_acc(finish(buf[c][c * L:(c + 1) * L], op, p), dtype) for c in range(p)])


def all_gather(shards):
    """All-gather: every rank receives the concatenation of the p shards."""
    shards = np.asarray(shards)
    p = shards.shape[0]
    full = np.concatenate([shards[c] for c in range(p)])
    return np.stack([full.copy() for _ in range(p)])


def fold_elements_ring_order(cols, chunk_of, op, dtype):
    """Ring-order fold of selected elements.

    ``cols`` has shape (p, m): the p ranks' values at m element positions;
    ``chunk_of`` (m,) gives the chunk each position lies in.  Position i of
    chunk c folds x_{c+1}, x_{c+2}, ..., x_c (mod p).  Returns (m,) results in
    the storage type.
    """
    cols = _check(cols, dtype, op)
    chunk_of = np.asarray(chunk_of, dtype=np.int64)
    p, m = cols.shape
    acc_rows = [to_acc(cols[r], dtype) for r in range(p)]
    res = to_acc(cols[0], dtype)
    for c in np.unique(chunk_of):
        sel = chunk_of == c
        acc = acc_rows[(c + 1) % p][sel]
        for k in range(2, p + 1):
            acc = combine(acc, acc_rows[(c + k) % p][sel], op)
        res[sel] = finish(acc, op, p)
    return from_acc(res, dtype)


def all_reduce_fold(xs, op, dtype):
    """Ring all-reduce written as the per-chunk formula (independent of the
    schedule simulation): chunk c folds x_{c+1}, ..., x_c; every rank gets y."""
    xs = _check(xs, dtype, op)
    p, n = xs.shape
    b = chunk_bounds(n, p)
    y = np.empty(n, dtype=xs.dtype)
    for c in range(p):
        lo, hi = b[c], b[c + 1]
        acc = to_acc(xs[(c + 1) % p, lo:hi], dtype)
        for k in range(2, p + 1):
            acc = combine(acc, to_acc(xs[(c + k) % p, lo:hi], dtype), op)
        y[lo:hi] = from_acc(finish(acc, op, p), dtype)
    return np.stack([y.copy() for _ in range(p)])


def reduce(xs, op, dtype):
    """Reduce to one rank: ascending fold x_0, x_1, ..., x_{p-1}; shape (n,)."""
    xs = _check(xs, dtype, op)
    acc = to_acc(xs[0], dtype)
    for r in range(1, xs.shape[0]):
        acc = combine(acc, to_acc(xs[r], dtype), op)
    return from_acc(finish(acc, op, xs.shape[0]), dtype)


def broadcast(x, p):
    """Broadcast: every one of the p ranks receives a copy of the root's buffer."""
    x = np.asarray(x)
    return np.stack([x.copy() for _ in range(p)])


def all_reduce_hier(xs, op, dtype, group_size, intra="reduce", wire_round=False):
    """Hierarchical all-reduce in the steps of page "大模型并行的最小闭环",
    section "Source Log: 2026-05-05" (hierarchical AllReduce + SHARP).

    Step 1: inside each group the members' buffers are combined into the
    representative's partial, in the accumulator type.  intra="reduce" (the
    default reading) folds the members ascending; intra="ring" follows the
    page's wording of step 1 literally, an all-reduce inside the group, run as
    a ring of the G members (chunk k of the n elements folds members
    k+1, ..., k of the group, the order of ``all_reduce_fold``).  Step 2: the
    representative is the group's first rank.  wire_round=True rounds each
    group partial to the storage type at the representative (it crosses
    groups in that type) and widens it again.  Steps 3-4: the representatives'
    partials are combined (ascending over groups).  Step 5: the result goes
    back to every representative.  Step 6: each representative broadcasts it
    inside its group.  Returns the (p, n) outputs.
    """
    xs = _check(xs, dtype, op)
    p, n = xs.shape
    G = int(group_size)
    if G < 1 or p % G:
        raise ValueError("group_size must divide p")
    if intra not in ("reduce", "ring"):
        raise ValueError(f"unknown intra-group step {intra!r}")
    groups = [list(range(j * G, (j + 1) * G)) for j in range(p // G)]
    partial = []
    for members in groups:  # steps 1-2
        if intra == "reduce":
            acc = to_acc(xs[members[0]], dtype)
            for r in members[1:]:
                acc = combine(acc, to_acc(xs[r], dtype), op)
        else:
            acc = np.empty(n, dtype=to_acc(xs[0, :0], dtype).dtype)
            b = chunk_bounds(n, G)
            for k in range(G):
                lo, hi = b[k], b[k + 1]
                part = to_acc(xs[members[(k + 1) % G], lo:hi], dtype)
                for i in range(2, G + 1):
                    part = combine(part, to_acc(xs[members[(k + i) % G], lo:hi], dtype), op)
                acc[lo:hi] = part
        if wire_round:
            acc = to_acc(from_acc(acc, dtype), dtype)
        partial.append(acc)
    total = partial[0]  # steps 3-4
    for g in partial[1:]:
        total = combine(total, g, op)
    result = from_acc(finish(total, op, p), dtype)
    out = np.empty_like(xs)
    for members in groups:  # steps 5-6
        for r in members:
            out[r] = result
    return out


def scatter(x, p):
    """Scatter (page "分布式训练/推理", section "通信原语"): the root splits its
    tensor into p equal slices and rank c receives slice c.  Returns (p, n/p)."""
    x = np.asarray(x)
    n = x.shape[0]
    if n % p:
        raise ValueError("scatter needs p | n")
    L = n // p
    return np.stack([x[c * L:(c + 1) * L].copy() for c in range(p)])


def gather(shards):
    """Gather (same section): the p ranks' slices are collected, in rank
    order, at one rank.  Returns the (p*L,) concatenation."""
    shards = np.asarray(shards)
    return np.concatenate([shards[c] for c in range(shards.shape[0])])


def all_reduce_bucket(tensors, op, dtype):
    """Bucketed all-reduce (page "分布式训练/推理", section on gradient
    synchronisation: the gradients are flattened into one bucket and
    all-reduced once).  ``tensors`` is a list of (p, n_j) arrays, tensor j of
    every rank; the bucket of rank r is the concatenation of its tensors in
    list order, the ring chunks the bucket, and the result is split back.
    Returns the list of (p, n_j) results."""
    tensors = [_check(t, dtype, op) for t in tensors]
    p = tensors[0].shape[0]
    bucket = np.concatenate(tensors, axis=1)
    red = all_reduce_fold(bucket, op, dtype)
    out, o = [], 0
    for t in tensors:
        out.append(red[:, o:o + t.shape[1]].copy())
        o += t.shape[1]
    return out


def all_gather_dim1(shards):
    """Tensor-parallel all-gather along the feature dimension (page
    "分布式训练/推理", tensor-parallel section: every rank's [B, d/p] output is
    gathered and concatenated along dim 1).  ``shards`` is (p, B, w); returns
    (p, B, p*w), the same [B, p*w] matrix on every rank."""
    shards = np.asarray(shards)
    p = shards.shape[0]
    full = np.concatenate([shards[c] for c in range(p)], axis=1)
    return np.stack([full.copy() for _ in range(p)])


def reduce_scatter_cols(xs, op, dtype):
    """Reduce-scatter of row-major [B, D] partial outputs along the feature
    dimension (the scatter strategy of the same section: the partial outputs
    are summed and rank j keeps output slice j, the psum_scatter).  ``xs`` is
    (p, B, D) with p | D; column block c = [c*D/p, (c+1)*D/p) is chunk c of
    the ring, folded x_{c+1}, ..., x_c as in ``reduce_scatter_ring``; rank c
    receives block c.  Returns (p, B, D/p)."""
    xs = np.asarray(xs)
    if xs.ndim != 3:
        raise ValueError("xs must have shape (p, B, D)")
    p, B, D = xs.shape
    if D % p:
        raise ValueError("the feature dimension must be divisible by p")
    w = D // p
    _check(xs.reshape(p, B * D), dtype, op)
    out = []
    for c in range(p):
        acc = to_acc(xs[(c + 1) % p, :, c * w:(c + 1) * w], dtype)
        for k in range(2, p + 1):
            acc = combine(acc, to_acc(xs[(c + k) % p, :, c * w:(c + 1) * w], dtype), op)
        out.append(from_acc(finish(acc, op, p), dtype))
    return np.stack(out)
