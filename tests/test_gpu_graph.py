"""Graph capture of the collectives (calls through the C ABI, captured with
torch.cuda.graph and replayed).

A graph replays its kernel arguments unchanged, so launches whose
synchronisation state is tagged per launch (the phased fold's soft barrier,
the persistent ring executor's step flags) take a fixed tag under capture and
capture a reset of that state ahead of themselves.  Every case is replayed
several times on new inputs written into the captured buffers, with the same
collective run eagerly on the same stream between the replays (eager launches
carry fresh tags on the same slots), and every replay and every eager result
is compared bit for bit with the oracle.
"""

import pytest

import workloads as W
from gpu_util import assert_bitwise, to_dev, to_host, torch_dtype
from oracle import collectives as C

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def rr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import collective_communication_reduction_way_amd as mod

    mod.lib()
    return mod


def capture(fn):
    """Warm fn up on a side stream (first-call set-up stays out of the graph),
    then capture one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def load(dst, arr, dtype):
    """Write a host array into an existing device tensor (the captured address)."""
    dst.copy_(to_dev(arr, dtype).reshape(dst.shape))


def replay_and_check(rr, g, inputs, outputs, eager, make, dtype, what):
    """For each seed: new inputs into the captured buffers, replay, then the
    eager call into its own outputs; both against the oracle."""
    t0 = rr.barrier_timeouts()
    f0 = rr.ring_exec_failures()
    for k in range(REPLAYS):
        xs, want = make(100 + k)
        for buf, arr in zip(inputs, xs):
            load(buf, arr, dtype)
        for o in outputs:
            o.fill_(0)
        g.replay()
        eager_outs = eager()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outputs, want)):
            assert_bitwise(to_host(o, dtype).reshape(w.shape), w, f"{what}: replay {k}, output {i}")
        for i, (o, w) in enumerate(zip(eager_outs, want)):
            assert_bitwise(to_host(o, dtype).reshape(w.shape), w, f"{what}: eager after replay {k}, output {i}")
    assert rr.barrier_timeouts() == t0, f"{what}: a soft barrier timed out"
    assert rr.ring_exec_failures() == f0, f"{what}: an executor wait timed out"


def inputs_for(seed, p, n, dtype):
    return W.random_inputs(seed, p, n, dtype, kind="full" if dtype == "int32" else "normal")


AR_CASES = [
    # (algo, group, dtype, p, n, op): single round, several rounds (the
    # barrier), 16-bit, ragged, staged, hierarchical, persistent executor
    ("ring", 0, "float32", 8, 2097152, "sum"),
    ("ring", 0, "float32", 8, 8388608, "sum"),
    ("ring", 0, "bfloat16", 8, 16777216 + 24, "avg"),
    ("ring", 0, "int32", 5, 100003, "max"),
    ("ring_staged", 0, "bfloat16", 8, 262144 + 7, "sum"),
    ("hier", 4, "bfloat16", 8, 16777216, "sum"),
    ("hier_staged", 2, "float32", 8, 1048576 + 3, "min"),
    ("ring_persistent", 0, "float32", 8, 2097152, "sum"),
    ("ring_persistent", 0, "bfloat16", 4, 100003, "sum"),
    ("ring_persistent", 0, "float16", 8, 1 << 20, "avg"),
]


@pytest.mark.parametrize("case", range(len(AR_CASES)))
def test_all_reduce_graph(rr, case):
    algo, G, dtype, p, n, op = AR_CASES[case]

    def make(seed):
        x = inputs_for(seed, p, n, dtype)
        if algo.startswith("hier"):
            w = C.all_reduce_hier(x, op, dtype, G)
        else:
            w = C.all_reduce_ring(x, op, dtype)
        return [x], [w]

    tdt = torch_dtype(dtype)
    xs = torch.zeros((p, n), dtype=tdt, device="cuda")
    ys = torch.zeros((p, n), dtype=tdt, device="cuda")
    ye = torch.zeros((p, n), dtype=tdt, device="cuda")
    need = rr.workspace_size(algo, p, G, n, tdt)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    wse = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    call = lambda out, w: rr.all_reduce(xs, out, op=op, algo=algo, group_size=G, workspace=w if need else None)
    load(xs, make(99)[0][0], dtype)
    g = capture(lambda: call(ys, ws))
    replay_and_check(rr, g, [xs], [ys], lambda: (call(ye, wse), [ye])[1], make, dtype,
                     f"{algo} {dtype} p={p} n={n} {op}")
    del g
    torch.cuda.empty_cache()


def test_hier_variants_graph(rr):
    """The hierarchical variants (intra-group ring, wire rounding), several rounds."""
    p, n, G, dtype = 8, 16777216 + 5, 4, "bfloat16"
    tdt = torch_dtype(dtype)
    xs = torch.zeros((p, n), dtype=tdt, device="cuda")
    ys = torch.zeros_like(xs)
    ye = torch.zeros_like(xs)
    for kw in (dict(intra="ring"), dict(wire_round=True), dict(intra="ring", wire_round=True)):
        def make(seed, kw=kw):
            x = inputs_for(seed, p, n, dtype)
            return [x], [C.all_reduce_hier(x, "sum", dtype, G, **kw)]

        load(xs, make(99)[0][0], dtype)
        g = capture(lambda kw=kw: rr.all_reduce_hier(xs, ys, op="sum", group_size=G, **kw))
        replay_and_check(rr, g, [xs], [ys], lambda kw=kw: (rr.all_reduce_hier(xs, ye, group_size=G, **kw), [ye])[1],
                         make, dtype, f"hier {kw}")
        del g
    torch.cuda.empty_cache()


def test_rs_ag_reduce_broadcast_graph(rr):
    """A sequence in one graph: reduce-scatter, all-gather of its shards,
    reduce to a root and broadcast of the root's result (32 MiB per rank:
    reduce-scatter and reduce take the batched rounds behind the barrier)."""
    p, n, dtype = 8, 8 * 1048576 + 8 * 3, "float32"
    L = n // p
    tdt = torch_dtype(dtype)
    xs = torch.zeros((p, n), dtype=tdt, device="cuda")
    sh = torch.zeros((p, L), dtype=tdt, device="cuda")
    ag = torch.zeros((p, n), dtype=tdt, device="cuda")
    red = torch.zeros((n,), dtype=tdt, device="cuda")
    bc = torch.zeros((p, n), dtype=tdt, device="cuda")
    e_sh, e_ag, e_red, e_bc = (torch.zeros_like(t) for t in (sh, ag, red, bc))

    def seq(sh, ag, red, bc):
        rr.reduce_scatter(xs, sh)
        rr.all_gather(sh, ag)
        rr.reduce(xs, red, root=3)
        rr.broadcast(red, bc, root=3)

    def make(seed):
        x = inputs_for(seed, p, n, dtype)
        rs = C.reduce_scatter_ring(x, "sum", dtype)
        r = C.reduce(x, "sum", dtype)
        return [x], [rs, C.all_gather(rs), r, C.broadcast(r, p)]

    load(xs, make(99)[0][0], dtype)
    g = capture(lambda: seq(sh, ag, red, bc))
    replay_and_check(rr, g, [xs], [sh, ag, red, bc], lambda: (seq(e_sh, e_ag, e_red, e_bc), [e_sh, e_ag, e_red, e_bc])[1],
                     make, dtype, "rs/ag/reduce/broadcast")
    del g
    torch.cuda.empty_cache()


def test_bucket_and_tp_layouts_graph(rr):
    """The bucketed all-reduce and the dim-1 reduce-scatter / all-gather."""
    p, dtype = 8, "bfloat16"
    tdt = torch_dtype(dtype)
    sizes = [1000, 65536 + 12, 3, 768 * 768]
    parts = [torch.zeros((p, m), dtype=tdt, device="cuda") for m in sizes]
    outs = [torch.zeros_like(t) for t in parts]
    eouts = [torch.zeros_like(t) for t in parts]
    rows, w = 33, 64
    mat = torch.zeros((p, rows, p * w), dtype=tdt, device="cuda")
    rs = torch.zeros((p, rows, w), dtype=tdt, device="cuda")
    agm = torch.zeros((p, rows, p * w), dtype=tdt, device="cuda")
    e_rs, e_agm = torch.zeros_like(rs), torch.zeros_like(agm)

    def seq(outs, rs, agm):
        rr.all_reduce_bucket(parts, outs, op="sum")
        rr.reduce_scatter_dim1(mat, rs)
        rr.all_gather_dim1(rs, agm)

    def make(seed):
        xs = [inputs_for(seed + 7 * i, p, m, dtype) for i, m in enumerate(sizes)]
        xm = inputs_for(seed + 50, p, rows * p * w, dtype).reshape(p, rows, p * w)
        want = C.all_reduce_bucket(xs, "sum", dtype)
        cols = C.reduce_scatter_cols(xm, "sum", dtype)
        return xs + [xm], want + [cols, C.all_gather_dim1(cols)]

    first = make(99)[0]
    for buf, arr in zip(parts + [mat], first):
        load(buf, arr, dtype)
    g = capture(lambda: seq(outs, rs, agm))
    replay_and_check(rr, g, parts + [mat], outs + [rs, agm], lambda: (seq(eouts, e_rs, e_agm), eouts + [e_rs, e_agm])[1],
                     make, dtype, "bucket + dim-1 layouts")
    del g
    torch.cuda.empty_cache()


def test_executor_graphs_replayed_concurrently(rr):
    """Two graphs, each holding one persistent-executor all-reduce, captured
    one after the other (on the same capture stream), then replayed at the
    same time on two different streams, three times: each captured launch
    owns its own step flags, so neither replay's flag reset or flags disturb
    the other, and both give the oracle's bits with no wait timing out."""
    p, n, dtype = 4, 65536 + 5, "float32"
    tdt = torch_dtype(dtype)
    xa, xb = (torch.zeros((p, n), dtype=tdt, device="cuda") for _ in range(2))
    ya, yb = torch.zeros_like(xa), torch.zeros_like(xb)
    ga = capture(lambda: rr.all_reduce(xa, ya, algo="ring_persistent"))
    gb = capture(lambda: rr.all_reduce(xb, yb, algo="ring_persistent"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    f0 = rr.ring_exec_failures()
    for k in range(REPLAYS):
        x1, x2 = inputs_for(200 + k, p, n, dtype), inputs_for(300 + k, p, n, dtype)
        load(xa, x1, dtype)
        load(xb, x2, dtype)
        ya.fill_(0)
        yb.fill_(0)
        torch.cuda.synchronize()
        # both streams start after the same short spin, so the replays overlap
        for s, g in ((s1, ga), (s2, gb)):
            with torch.cuda.stream(s):
                torch.cuda._sleep(2_000_000)
                g.replay()
        torch.cuda.synchronize()
        assert_bitwise(to_host(ya, dtype), C.all_reduce_ring(x1, "sum", dtype), f"graph a, replay {k}")
        assert_bitwise(to_host(yb, dtype), C.all_reduce_ring(x2, "sum", dtype), f"graph b, replay {k}")
    assert rr.ring_exec_failures() == f0, "an executor wait timed out"
    del ga, gb
    torch.cuda.empty_cache()
