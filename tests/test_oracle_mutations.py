"""Plant plausible mistakes in the CPU oracle and check that its pins catch
every one (a pin set that a dropped term, a swapped operand, a wrong index or
a wrong rounding can pass would not be pinning anything).  CPU only; the
mistakes live in monkeypatched copies of oracle functions for one test."""

import numpy as np
import pytest

import oracle_pins as P
from oracle import bf16 as B
from oracle import collectives as C
from oracle import cost as K
from oracle import fp16 as H

_combine = C.combine
_narrow = B.narrow
_to_acc = C.to_acc
_finish = C.finish
_hier = C.all_reduce_hier
_fold = C.all_reduce_fold
_h_narrow = H.narrow
_ulp = B.ulp_distance


def _ulp_key(key):
    """An ulp distance built on another 16-bit key (planted mistakes)."""
    return lambda a, b: np.abs(key(np.asarray(a, dtype=np.uint16).astype(np.int64)) -
                               key(np.asarray(b, dtype=np.uint16).astype(np.int64)))


def _run_all_pins():
    """Return the names of the pins that fail."""
    failed = []
    checks = [
        ("worked_example", lambda: [P.pin_worked_example(d) for d in C.DTYPES]),
        ("worked_example_max_min", lambda: [P.pin_worked_example_max_min(d) for d in C.DTYPES]),
        ("closed_form", lambda: [P.pin_closed_form(p, n, d) for d in C.DTYPES for p, n in ((3, 100), (8, 4099))]),
        ("ring_order_probe", lambda: [P.pin_ring_order_probe(d) for d in ("float32", "bfloat16")]),
        ("reduce_order_probe", lambda: [P.pin_reduce_order_probe(d) for d in ("float32", "bfloat16")]),
        ("hier_probe", lambda: [P.pin_hier_probe(d) for d in ("float32", "bfloat16")]),
        ("bf16_hand", P.pin_bf16_rounding_hand),
        ("bf16_nan", P.pin_bf16_nan),
        ("bf16_ulp", lambda: P.pin_bf16_ulp_distance(count=1 << 12)),
        ("bf16_torch", lambda: P.pin_bf16_vs_torch(count=1 << 18)),
        ("int32_wrap", P.pin_int32_wrap),
        ("signed_zero", P.pin_max_min_signed_zero),
        ("bruteforce_int", lambda: P.pin_bruteforce_int(0)),
        ("bruteforce_float", lambda: P.pin_bruteforce_float(0)),
        ("identities", lambda: P.pin_identities(3)),
        ("schedule", lambda: [P.pin_schedule_symbolic(p) for p in (2, 3, 4, 8)]),
        ("hier_vs_flat", lambda: P.pin_hier_vs_flat(1)),
        ("edge_cases", P.pin_edge_cases),
        ("fp16_hand", P.pin_fp16_rounding_hand),
        ("fp16_numpy", lambda: P.pin_fp16_vs_numpy(count=1 << 18)),
        ("fp16_order", P.pin_fp16_order_probes),
        ("fp16_once", P.pin_fp16_sum_rounds_once),
        ("avg_worked", P.pin_avg_worked_example),
        ("avg_closed_form", lambda: [P.pin_avg_closed_form(p, n) for p, n in ((3, 100), (8, 4099))]),
        ("avg_probes", P.pin_avg_division_probes),
        ("avg_rounded", lambda: P.pin_avg_correctly_rounded(0)),
        ("avg_ring_int", P.pin_avg_ring_order_and_int),
        ("scatter_gather", P.pin_scatter_gather),
        ("bucket", P.pin_bucket),
        ("ag_dim1", P.pin_all_gather_dim1),
        ("rs_cols", P.pin_reduce_scatter_cols),
        ("hier_variants", P.pin_hier_variants),
        ("cost_ring", P.pin_cost_ring),
        ("cost_hier", P.pin_cost_hier_example),
    ]
    for name, fn in checks:
        try:
            with np.errstate(all="ignore"):
                fn()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(name)
    return failed


def _sched_rs_off_by_one(p):
    out = []
    for s in range(p - 1):
        for r in range(p):
            out.append(("rs", s, r, (r + 1) % p, (r - s) % p))
    for s in range(p - 1):
        for r in range(p):
            out.append(("ag", s, r, (r + 1) % p, (r - s) % p))
    return out


def _sched_backwards(p):
    out = []
    for s in range(p - 1):
        for r in range(p):
            out.append(("rs", s, r, (r - 1) % p, (r + 1 + s) % p))
    for s in range(p - 1):
        for r in range(p):
            out.append(("ag", s, r, (r - 1) % p, (r + s) % p))
    return out


def _fold_from_c(xs, op, dtype):
    xs = np.asarray(xs)
    p, n = xs.shape
    b = C.chunk_bounds(n, p)
    y = np.empty(n, dtype=xs.dtype)
    for c in range(p):
        lo, hi = b[c], b[c + 1]
        acc = C.to_acc(xs[c % p, lo:hi], dtype)
        for k in range(1, p):
            acc = C.combine(acc, C.to_acc(xs[(c + k) % p, lo:hi], dtype), op)
        y[lo:hi] = C.from_acc(acc, dtype)
    return np.stack([y.copy() for _ in range(p)])


def _reduce_descending(xs, op, dtype):
    xs = np.asarray(xs)
    acc = C.to_acc(xs[-1], dtype)
    for r in range(xs.shape[0] - 2, -1, -1):
        acc = C.combine(acc, C.to_acc(xs[r], dtype), op)
    return C.from_acc(acc, dtype)


def _hier_strided(xs, op, dtype, group_size):
    xs = np.asarray(xs)
    p, n = xs.shape
    G = group_size
    ng = p // G
    parts = []
    for j in range(ng):
        members = list(range(j, p, ng))
        acc = C.to_acc(xs[members[0]], dtype)
        for r in members[1:]:
            acc = C.combine(acc, C.to_acc(xs[r], dtype), op)
        parts.append(acc)
    t = parts[0]
    for g in parts[1:]:
        t = C.combine(t, g, op)
    return np.stack([C.from_acc(t, dtype)] * p)


def _hier_round_at_rep(xs, op, dtype, group_size):
    xs = np.asarray(xs)
    p, n = xs.shape
    G = group_size
    parts = []
    for j in range(p // G):
        acc = C.to_acc(xs[j * G], dtype)
        for r in range(j * G + 1, (j + 1) * G):
            acc = C.combine(acc, C.to_acc(xs[r], dtype), op)
        parts.append(C.to_acc(C.from_acc(acc, dtype), dtype))
    t = parts[0]
    for g in parts[1:]:
        t = C.combine(t, g, op)
    return np.stack([C.from_acc(t, dtype)] * p)


def _narrow_truncate(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def _narrow_ties_away(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x8000)) >> 16
    return np.where(is_nan, (u >> 16) | 0x40, r).astype(np.uint16)


def _narrow_no_quiet(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _h_truncate(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.int64)
    sign = (u >> 16) & 0x8000
    a = u & 0x7FFFFFFF
    e = (a >> 23) - 112
    r = np.where(e > 0, (e << 10) | ((a & 0x7FFFFF) >> 13), 0)
    r = np.where(e >= 31, 0x7C00, r)
    return (sign | r).astype(np.uint16)


def _h_flush_subnormals(f):
    h = _h_narrow(f)
    return np.where((h & 0x7C00) == 0, h & 0x8000, h).astype(np.uint16)


def _h_ties_away(f):
    f = np.ascontiguousarray(f, dtype=np.float32).astype(np.float64)
    # round half away from zero at the binary16 grid (normal range only)
    m, e = np.frexp(np.abs(f))
    q = np.floor(np.abs(f) / np.exp2(e - 11) + 0.5) * np.exp2(e - 11)
    return (np.sign(f) * q).astype(np.float16).view(np.uint16)


def _bucket_per_tensor(tensors, op, dtype):
    return [C.all_reduce_fold(np.asarray(t), op, dtype) for t in tensors]


def _ag_dim1_rows(shards):
    shards = np.asarray(shards)
    p, B_, w = shards.shape
    full = np.concatenate(list(shards), axis=0).reshape(B_, p * w)
    return np.stack([full] * p)


def _rs_cols_ascending(xs, op, dtype):
    xs = np.asarray(xs)
    p, B_, D = xs.shape
    w = D // p
    out = []
    for c in range(p):
        acc = C.to_acc(xs[0, :, c * w:(c + 1) * w], dtype)
        for r in range(1, p):
            acc = C.combine(acc, C.to_acc(xs[r, :, c * w:(c + 1) * w], dtype), op)
        out.append(C.from_acc(C.finish(acc, op, p), dtype))
    return np.stack(out)


def _rs_cols_row_major_chunks(xs, op, dtype):
    xs = np.asarray(xs)
    p, B_, D = xs.shape
    flat = C.reduce_scatter_ring(xs.reshape(p, B_ * D), op, dtype)
    return flat.reshape(p, B_, D // p)


def _to_acc_int_as_float(x, dtype):
    if dtype == "int32":
        return np.asarray(x).astype(np.float32)
    return _to_acc(x, dtype)


MUTATIONS = {
    "rs_chunk_off_by_one": lambda m: m.setattr(C, "ring_schedule", _sched_rs_off_by_one),
    "ring_runs_backwards": lambda m: m.setattr(C, "ring_schedule", _sched_backwards),
    "receiver_folds_local_first": lambda m: m.setattr(C, "combine", lambda a, v, op: _combine(v, a, op)),
    "max_min_non_strict": lambda m: m.setattr(
        C, "combine", lambda a, v, op: np.where(v >= a, v, a) if op == "max" else
        (np.where(v <= a, v, a) if op == "min" else _combine(a, v, op))),
    "sum_drops_a_term": lambda m: m.setattr(
        C, "combine", lambda a, v, op: a if (op == "sum" and np.size(a) % 3 == 1) else _combine(a, v, op)),
    "max_min_swapped": lambda m: m.setattr(
        C, "combine", lambda a, v, op: _combine(a, v, {"max": "min", "min": "max"}.get(op, op))),
    "fold_starts_at_own_rank": lambda m: m.setattr(C, "all_reduce_fold", _fold_from_c),
    "reduce_descending": lambda m: m.setattr(C, "reduce", _reduce_descending),
    "hier_groups_strided": lambda m: m.setattr(C, "all_reduce_hier", _hier_strided),
    "hier_rounds_at_representative": lambda m: m.setattr(C, "all_reduce_hier", _hier_round_at_rep),
    "bf16_truncates": lambda m: m.setattr(B, "narrow", _narrow_truncate),
    "bf16_ties_away": lambda m: m.setattr(B, "narrow", _narrow_ties_away),
    "bf16_nan_not_quieted": lambda m: m.setattr(B, "narrow", _narrow_no_quiet),
    "int32_accumulates_in_float": lambda m: m.setattr(C, "to_acc", _to_acc_int_as_float),
    "chunk_bounds_ceil": lambda m: m.setattr(C, "chunk_bounds", lambda n, p: [-((-c * n) // p) for c in range(p + 1)]),
    "avg_multiplies_by_reciprocal": lambda m: m.setattr(
        C, "finish", lambda a, op, p: a * (np.float32(1) / np.float32(p)) if op == "avg" else a),
    "avg_not_divided": lambda m: m.setattr(C, "finish", lambda a, op, p: a),
    "avg_divides_by_p_minus_1": lambda m: m.setattr(
        C, "finish", lambda a, op, p: a / np.float32(max(p - 1, 1)) if op == "avg" else a),
    "avg_rounds_sum_first": lambda m: m.setattr(
        C, "finish", lambda a, op, p: (B.widen(B.narrow(a)) / np.float32(p)).astype(np.float32)
        if op == "avg" else a),
    "fp16_truncates": lambda m: m.setattr(H, "narrow", _h_truncate),
    "fp16_flushes_subnormals": lambda m: m.setattr(H, "narrow", _h_flush_subnormals),
    "fp16_ties_away": lambda m: m.setattr(H, "narrow", _h_ties_away),
    "bucket_chunked_per_tensor": lambda m: m.setattr(C, "all_reduce_bucket", _bucket_per_tensor),
    "all_gather_dim1_as_rows": lambda m: m.setattr(C, "all_gather_dim1", _ag_dim1_rows),
    "reduce_scatter_cols_ascending": lambda m: m.setattr(C, "reduce_scatter_cols", _rs_cols_ascending),
    "reduce_scatter_cols_row_major": lambda m: m.setattr(C, "reduce_scatter_cols", _rs_cols_row_major_chunks),
    "hier_ignores_intra_ring": lambda m: m.setattr(
        C, "all_reduce_hier", lambda xs, op, dt, G, intra="reduce", wire_round=False: _hier(xs, op, dt, G, "reduce",
                                                                                           wire_round)),
    "hier_ignores_wire_round": lambda m: m.setattr(
        C, "all_reduce_hier", lambda xs, op, dt, G, intra="reduce", wire_round=False: _hier(xs, op, dt, G, intra)),
    "scatter_reversed": lambda m: m.setattr(
        C, "scatter", lambda x, p: np.stack([np.asarray(x)[c * (len(x) // p):(c + 1) * (len(x) // p)]
                                              for c in range(p)][::-1])),
    "cost_ring_p_rounds": lambda m: m.setattr(
        K, "ring_all_reduce", lambda p, nb, a, bw: 2 * p * (a + nb / p / bw)),
    "cost_ring_full_message": lambda m: m.setattr(
        K, "ring_all_reduce", lambda p, nb, a, bw: 2 * (p - 1) * (a + nb / bw)),
    "cost_hier_links_swapped": lambda m: m.setattr(
        K, "hier_all_reduce", lambda G, nb, fast, slow: (K.message(*fast, G * nb),
                                                         K.message(*slow, G * nb) + K.message(*fast, nb))),
    "cost_hier_ships_node_bytes": lambda m: m.setattr(
        K, "hier_all_reduce", lambda G, nb, fast, slow: (K.message(*slow, G * nb),
                                                         K.message(*fast, G * nb) + K.message(*slow, G * nb))),
    "ulp_signed_zero_apart": lambda m: m.setattr(B, "ulp_distance", _ulp_key(
        lambda h: np.where(h & 0x8000, -(h & 0x7FFF) - 1, h & 0x7FFF))),
    "ulp_sign_ignored": lambda m: m.setattr(B, "ulp_distance", _ulp_key(lambda h: h & 0x7FFF)),
    "ulp_unsigned_pattern": lambda m: m.setattr(B, "ulp_distance", _ulp_key(lambda h: h)),
    "ulp_one_step_short": lambda m: m.setattr(B, "ulp_distance", lambda a, b: np.maximum(
        _ulp(a, b) - (_ulp(a, b) > 1), 0)),
    "all_gather_reversed": lambda m: m.setattr(
        C, "all_gather", lambda sh: np.stack([np.concatenate(list(np.asarray(sh))[::-1])] * np.asarray(sh).shape[0])),
}


def test_unmutated_oracle_passes_every_pin():
    assert _run_all_pins() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    MUTATIONS[name](monkeypatch)
    failed = _run_all_pins()
    assert failed, f"planted mistake {name!r} passed every pin"
