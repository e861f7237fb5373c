"""GPU parity of the hierarchical all-reduce's variants against the CPU
oracle (calls go through the C ABI): step 1 as a ring all-reduce inside each
group (intra="ring"), group partials rounded to the storage type before the
cross-group fold (wire_round), and the staged execution of both.  Bit for
bit: both sides take the same fold order and the same roundings.
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
VARIANTS = (dict(intra="ring"), dict(wire_round=True), dict(intra="ring", wire_round=True),
            dict(wire_round=True, staged=True), dict(staged=True))


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def run(rr, x, dtype, op, G, **kw):
    xs = to_dev(x, dtype)
    out = torch.empty_like(xs)
    rr.all_reduce_hier(xs, out, op=op, group_size=G, **kw)
    return to_host(out, dtype)


def want(x, dtype, op, G, intra="reduce", wire_round=False, staged=False):
    return C.all_reduce_hier(x, op, dtype, G, intra=intra, wire_round=wire_round)


def test_intra_ring_probe(rr):
    """With one group of 4 the intra-group ring is the ring all-reduce (the
    ring probe gives zeros; the ascending default gives [2, 2, 2, 0]); two
    groups holding the probe each also give zeros."""
    x = PIN.enc(PIN.ring_order_probe_inputs(), "float32")
    assert_bitwise(run(rr, x, "float32", "sum", 4, intra="ring"), np.zeros((4, 4), np.float32), "one group")
    assert_bitwise(run(rr, x, "float32", "sum", 4), np.stack([np.array([2, 2, 2, 0], np.float32)] * 4), "default")
    x8 = np.concatenate([x, x])
    assert_bitwise(run(rr, x8, "float32", "sum", 4, intra="ring"), np.zeros((8, 4), np.float32), "two groups")


@pytest.mark.parametrize("staged", (False, True))
def test_wire_round_probe(rr, staged):
    """bf16 x = [1, 2^-8, 2^-8, 0] in groups of 2: the partial 1 + 2^-8 rounds
    to 1 on the wire and the result is 1; float32 partials give 1 + 2^-7."""
    x = PIN.enc([[1.0], [2.0 ** -8], [2.0 ** -8], [0.0]], "bfloat16")
    got = run(rr, x, "bfloat16", "sum", 2, wire_round=True, staged=staged)
    assert np.all(got == 0x3F80), [hex(v) for v in got.ravel()]
    got = run(rr, x, "bfloat16", "sum", 2, staged=staged)
    assert np.all(got == 0x3F81), [hex(v) for v in got.ravel()]


SWEEP = [(2, 1000), (4, 65536 + 12), (6, 4099), (8, 131072 + 5), (8, 7), (16, 40000), (64, 640)]


@pytest.mark.parametrize("p,n", SWEEP)
@pytest.mark.parametrize("dtype", DTYPES)
def test_variants_sweep(rr, p, n, dtype):
    x = W.random_inputs(71, p, n, dtype, kind="full" if dtype == "int32" else "normal")
    ops = ("sum", "max", "min") + (("avg",) if dtype != "int32" else ())
    groups = [g for g in (1, 2, 3, 4, p) if p % g == 0]
    for G in groups:
        for kw in VARIANTS:
            for op in ops:
                assert_bitwise(run(rr, x, dtype, op, G, **kw), want(x, dtype, op, G, **kw), f"G={G} {kw} {op}")


@pytest.mark.parametrize("batch", ("0", "1"))
@pytest.mark.parametrize("dtype", ("float32", "bfloat16", "float16"))
def test_variants_multi_round(rr, tuning, dtype, batch):
    """Sizes that take several rounds of the phased fold (with its barrier),
    ragged group-chunk bounds, in batched rounds (batch 0, the default) and
    in single-tile rounds (batch 1)."""
    tuning.set("RR_AR_BATCH", batch)
    p = 8
    n = 8 * (1 << 20) * (2 if dtype != "float32" else 1) + 13
    x = W.random_inputs(72, p, n, dtype)
    t0 = rr.barrier_timeouts()
    for G in (2, 4):
        for kw in (dict(intra="ring"), dict(intra="ring", wire_round=True), dict(wire_round=True)):
            for op in ("sum", "avg"):
                assert_bitwise(run(rr, x, dtype, op, G, **kw), want(x, dtype, op, G, **kw), f"G={G} {kw} {op}")
    assert rr.barrier_timeouts() == t0
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ("float32", "float16"))
def test_variants_unaligned(rr, dtype):
    """Rank buffers one element off 16-byte alignment take the single-pass
    element path of the variants."""
    p, n = 4, 10007
    x = W.random_inputs(73, p, n + 3, dtype)
    base = to_dev(x, dtype)
    ins = [base[r, 1:1 + n] for r in range(p)]
    outbuf = torch.empty((p, n + 1), dtype=base.dtype, device="cuda")
    outs = [outbuf[r, 1:1 + n] for r in range(p)]
    shifted = np.ascontiguousarray(x[:, 1:1 + n])
    for kw in (dict(intra="ring"), dict(wire_round=True), dict(intra="ring", wire_round=True)):
        rr.all_reduce_hier(ins, outs, op="sum", group_size=2, **kw)
        got = np.stack([to_host(o, dtype) for o in outs])
        assert_bitwise(got, want(shifted, dtype, "sum", 2, **kw), f"{kw}")


def test_staged_intra_ring_is_unsupported(rr):
    xs = torch.ones((4, 64), dtype=torch.float32, device="cuda")
    out = torch.full_like(xs, 7.0)
    with pytest.raises(rr.RRError):
        rr.all_reduce_hier(xs, out, group_size=2, intra="ring", staged=True)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
