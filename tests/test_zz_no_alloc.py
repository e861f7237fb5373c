"""rr_all_reduce_ex_noalloc, the all-reduce that allocates nothing (its
workspace is the library's fixed device scratch), against rr_all_reduce_ex
with a caller workspace: both called through the C ABI, two calls in a row
per case -- the second smaller, so that it runs over what the first left in
the scratch -- and every output compared bit for bit with the other entry
point's and with the oracle's.  Also: a call whose workspace would exceed the
scratch is refused and writes nothing, and the persistent executor is
refused."""

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_bitwise, to_dev, to_host, torch_dtype
from oracle import collectives as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20
INVALID, UNSUPPORTED = 1, 2


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def ptrs(rr, t):
    return rr._ptr_array([t[r].data_ptr() for r in range(t.shape[0])])


def run_ex(rr, xs, algo, G, op, dtype):
    """rr_all_reduce_ex with a torch workspace of rr_workspace_size bytes."""
    p, n = xs.shape
    out = torch.full_like(xs, float("nan")) if dtype != "int32" else torch.full_like(xs, -1)
    need = rr.workspace_size(algo, p, G, n, xs.dtype)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = rr.lib().rr_all_reduce_ex(ptrs(rr, xs), ptrs(rr, out), p, n, rr.DTYPES[dtype], rr.OPS[op], rr.ALGOS[algo],
                                   G, ws.data_ptr() if need else None, need,
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, rr.lib().rr_last_error().decode()
    return out, ws


def run_noalloc(rr, xs, algo, G, op, dtype):
    p, n = xs.shape
    out = torch.full_like(xs, float("nan")) if dtype != "int32" else torch.full_like(xs, -1)
    st = rr.lib().rr_all_reduce_ex_noalloc(ptrs(rr, xs), ptrs(rr, out), p, n, rr.DTYPES[dtype], rr.OPS[op],
                                           rr.ALGOS[algo], G, torch.cuda.current_stream().cuda_stream)
    assert st == 0, rr.lib().rr_last_error().decode()
    return out


CASES = [
    # (algo, group, dtype, p, first n, second n, op)
    ("ring_staged", 0, "bfloat16", 8, SCRATCH // (8 * 4), 100003, "sum"),  # the first fills the scratch exactly
    ("ring_staged", 0, "float16", 5, 777777, 4099, "avg"),
    ("hier_staged", 4, "bfloat16", 8, 4194304, 65536 + 9, "sum"),
    ("hier_staged", 2, "float32", 6, (1 << 20) + 3, 1001, "max"),
    ("ring_staged", 0, "float32", 8, 1 << 20, 1000, "sum"),  # 4-byte types need no workspace
    ("ring", 0, "bfloat16", 8, 1 << 20, 77, "sum"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_caller_workspace(rr, case):
    algo, G, dtype, p, n1, n2, op = CASES[case]
    for k, n in enumerate((n1, n2)):
        assert n2 < n1
        x = W.random_inputs(500 + 10 * case + k, p, n, dtype)
        xs = to_dev(x, dtype)
        got = run_noalloc(rr, xs, algo, G, op, dtype)
        ref, ws = run_ex(rr, xs, algo, G, op, dtype)
        torch.cuda.synchronize()
        what = f"{algo} G={G} {dtype} p={p} n={n} {op} (call {k + 1})"
        assert_bitwise(to_host(got, dtype), to_host(ref, dtype), what + ": noalloc vs caller workspace")
        want = C.all_reduce_hier(x, op, dtype, G) if algo.startswith("hier") else C.all_reduce_fold(x, op, dtype)
        assert_bitwise(to_host(got, dtype), want, what + ": noalloc vs oracle")
        del xs, got, ref, ws
    torch.cuda.empty_cache()


def test_noalloc_refuses_what_does_not_fit(rr):
    """A workspace need above the scratch: refused before any launch (the
    outputs keep their NaNs); the persistent executor: refused."""
    p, n, dtype = 8, SCRATCH // (8 * 4) + 8, "bfloat16"
    tdt = torch_dtype(dtype)
    assert rr.workspace_size("ring_staged", p, 0, n, tdt) > SCRATCH
    xs = torch.ones((p, n), dtype=tdt, device="cuda")
    out = torch.full_like(xs, float("nan"))
    L = rr.lib()
    s = torch.cuda.current_stream().cuda_stream
    st = L.rr_all_reduce_ex_noalloc(ptrs(rr, xs), ptrs(rr, out), p, n, rr.DTYPES[dtype], rr.OPS["sum"],
                                    rr.ALGOS["ring_staged"], 0, s)
    assert st == INVALID and b"scratch" in L.rr_last_error()
    st = L.rr_all_reduce_ex_noalloc(ptrs(rr, xs), ptrs(rr, out), p, 1024, rr.DTYPES[dtype], rr.OPS["sum"],
                                    rr.ALGOS["ring_persistent"], 0, s)
    assert st == UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
