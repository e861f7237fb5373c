"""The C ABI of librr.so on the CPU: every symbol declared in include/rr.h is
exported, and every invalid-argument path returns its status before any HIP
call (the pointers below are never dereferenced, nothing is launched)."""

import ctypes
import os
import re

import pytest

import collective_communication_reduction_way_amd as rr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rr.h")

INVALID, UNSUPPORTED = 1, 2
FAKE = 1 << 40  # a 16-byte aligned address that is never touched


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("rr_all_reduce", "rr_reduce_scatter", "rr_all_gather", "rr_reduce", "rr_broadcast"):
        assert f in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(rr.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    L = rr.lib()
    assert b"gfx950" in L.rr_version()
    for st in range(4):
        assert L.rr_status_string(st)


def ptrs(base, p, stride):
    return rr._ptr_array([base + r * stride for r in range(p)])


def ar(p=4, n=1024, dt=1, op=0, algo=0, group=0, send=None, recv=None, ws=None, wsb=0):
    L = rr.lib()
    send = send if send is not None else ptrs(FAKE, p, 1 << 20)
    recv = recv if recv is not None else ptrs(FAKE + (1 << 30), p, 1 << 20)
    st = L.rr_all_reduce_ex(send, recv, p, n, dt, op, algo, group, ws, wsb, None)
    return st, L.rr_last_error().decode()


@pytest.mark.parametrize("p", [0, -1, 65, 1000])
def test_all_reduce_bad_p(p):
    st, msg = ar(p=p)
    assert st == INVALID and "p=" in msg


def test_all_reduce_unknown_dtype_and_op():
    assert ar(dt=7)[0] == UNSUPPORTED
    assert ar(op=9)[0] == UNSUPPORTED


def test_all_reduce_null_arrays_and_buffers():
    L = rr.lib()
    assert L.rr_all_reduce(None, ptrs(FAKE, 4, 1 << 20), 4, 16, 1, 0, None) == INVALID
    assert L.rr_all_reduce(ptrs(FAKE, 4, 1 << 20), None, 4, 16, 1, 0, None) == INVALID
    send = rr._ptr_array([FAKE, FAKE + 4096, 0, FAKE + 8192])
    st, msg = ar(send=send, n=16)
    assert st == INVALID and "NULL" in msg


def test_all_reduce_misaligned():
    send = rr._ptr_array([FAKE + 2, FAKE + 8192, FAKE + 16384, FAKE + 32768])
    st, msg = ar(send=send, n=16, dt=1)
    assert st == INVALID and "aligned" in msg
    # 2-byte alignment is enough for bf16
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    st2, msg2 = ar(send=send, recv=recv, n=16, dt=2, algo=99)  # stop at the algo check after alignment
    assert st2 == INVALID and "algo" in msg2


def test_all_reduce_overlapping_outputs():
    recv = rr._ptr_array([FAKE, FAKE + 64, FAKE + (1 << 20), FAKE + (2 << 20)])
    send = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    st, msg = ar(send=send, recv=recv, n=64)
    assert st == INVALID and "overlap" in msg


def test_all_reduce_output_overlaps_other_input():
    send = ptrs(FAKE, 4, 1 << 20)
    recv = rr._ptr_array([FAKE + (1 << 20), FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)])
    st, msg = ar(send=send, recv=recv, n=64)
    assert st == INVALID and "overlaps input" in msg


def test_all_reduce_partial_in_place_is_rejected():
    send = ptrs(FAKE, 4, 1 << 20)
    recv = rr._ptr_array([FAKE + 16, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)])
    st, _ = ar(send=send, recv=recv, n=64)
    assert st == INVALID


def test_n_zero_is_a_no_op():
    # fully valid arguments apart from n = 0: nothing is launched
    assert ar(n=0)[0] == 0
    L = rr.lib()
    assert L.rr_reduce_scatter(ptrs(FAKE, 4, 1 << 20), ptrs(FAKE, 4, 1 << 20), 4, 0, 1, 0, None) == 0
    assert L.rr_all_gather(ptrs(FAKE, 4, 1 << 20), ptrs(FAKE, 4, 1 << 20), 4, 0, 1, None) == 0
    assert L.rr_reduce(ptrs(FAKE, 4, 1 << 20), FAKE, 0, 4, 0, 1, 0, None) == 0
    assert L.rr_broadcast(FAKE, ptrs(FAKE, 4, 1 << 20), 0, 4, 0, 1, None) == 0


def test_n_too_large():
    st, msg = ar(n=(1 << 56) + 1)
    assert st == INVALID and "2^56" in msg


@pytest.mark.parametrize("algo,group", [(2, 0), (2, 3), (2, 5), (3, 9), (3, -1)])
def test_hier_bad_group(algo, group):
    st, msg = ar(p=8, algo=algo, group=group)
    assert st == INVALID and "group_size" in msg


def test_unknown_algo():
    assert ar(algo=9)[0] == INVALID
    assert ar(algo=-1)[0] == INVALID


def test_persistent_ring_validation():
    """The persistent ring executor needs the staged ring's workspace for
    16-bit dtypes and none for 4-byte ones; every error path returns before
    any launch."""
    L = rr.lib()
    for dt in (2, 3):
        st, msg = ar(p=8, n=1024, dt=dt, algo=4)
        assert st == INVALID and "workspace" in msg
        assert L.rr_workspace_size(4, 8, 0, 1024, dt) == 8 * 1024 * 4
    assert L.rr_workspace_size(4, 8, 0, 1024, 1) == 0
    assert ar(algo=4, p=0)[0] == INVALID
    assert ar(algo=4, dt=0, op=3)[0] == UNSUPPORTED
    assert ar(algo=4, n=0)[0] == 0


def test_staged_workspace_required():
    st, msg = ar(p=8, n=1024, dt=2, algo=1)
    assert st == INVALID and "workspace" in msg
    need = rr.lib().rr_workspace_size(1, 8, 0, 1024, 2)
    assert need == 8 * 1024 * 4
    st, msg = ar(p=8, n=1024, dt=2, algo=1, ws=FAKE + (4 << 30), wsb=need - 1)
    assert st == INVALID and "smaller" in msg
    st, msg = ar(p=8, n=1024, dt=2, algo=1, ws=FAKE + (4 << 30) + 8, wsb=need)
    assert st == INVALID and "aligned" in msg
    # workspace overlapping an output
    st, msg = ar(p=8, n=1024, dt=2, algo=1, ws=FAKE + (1 << 30), wsb=need)
    assert st == INVALID and "workspace overlaps" in msg


def test_workspace_sizes():
    L = rr.lib()
    assert L.rr_workspace_size(0, 8, 0, 1000, 1) == 0
    assert L.rr_workspace_size(2, 8, 4, 1000, 2) == 0
    assert L.rr_workspace_size(1, 8, 0, 1000, 1) == 0
    assert L.rr_workspace_size(1, 8, 0, 1000, 0) == 0
    assert L.rr_workspace_size(1, 8, 0, 1000, 2) == 8 * 1000 * 4
    assert L.rr_workspace_size(3, 8, 4, 1000, 2) == 2 * 1000 * 4
    assert L.rr_workspace_size(3, 8, 2, 1000, 0) == 4 * 1000 * 4
    assert L.rr_workspace_size(3, 8, 3, 1000, 0) == 0  # invalid group
    # the staged hierarchy's group partials each start on a 16-byte boundary
    assert L.rr_workspace_size(3, 8, 4, 1001, 2) == 2 * 4016
    assert L.rr_workspace_size(3, 6, 2, 4099, 1) == 3 * 16400


def test_reduce_scatter_validation():
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    assert L.rr_reduce_scatter(send, recv, 4, 1001, 1, 0, None) == INVALID  # p does not divide n
    assert b"p | n" in L.rr_last_error()
    assert L.rr_reduce_scatter(send, recv, 4, 1024, 5, 0, None) == UNSUPPORTED
    assert L.rr_reduce_scatter(send, recv, 4, 1024, 1, 5, None) == UNSUPPORTED
    # output overlapping another rank's input
    bad = rr._ptr_array([FAKE + (1 << 20), FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)])
    assert L.rr_reduce_scatter(send, bad, 4, 1024, 1, 0, None) == INVALID
    # in place at the wrong slot (slot of chunk 0 for rank 1)
    bad2 = rr._ptr_array([FAKE + (5 << 30), FAKE + (1 << 20), FAKE + (2 << 30), FAKE + (3 << 30)])
    assert L.rr_reduce_scatter(send, bad2, 4, 1024, 1, 0, None) == INVALID


def test_all_gather_validation():
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    assert L.rr_all_gather(send, recv, 4, 1001, 1, None) == INVALID
    assert L.rr_all_gather(send, recv, 4, 1024, 7, None) == UNSUPPORTED
    # a shard inside another rank's output
    bad = rr._ptr_array([FAKE + (1 << 30) + (1 << 20), FAKE + (6 << 30), FAKE + (7 << 30), FAKE + (8 << 30)])
    assert L.rr_all_gather(bad, recv, 4, 1024, 1, None) == INVALID


def test_reduce_validation():
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    for root in (-1, 4):
        assert L.rr_reduce(send, FAKE + (1 << 30), root, 4, 64, 1, 0, None) == INVALID
    assert L.rr_reduce(send, 0, 0, 4, 64, 1, 0, None) == INVALID
    # output on a non-root input
    assert L.rr_reduce(send, FAKE + (1 << 20), 0, 4, 64, 1, 0, None) == INVALID
    assert L.rr_reduce(send, FAKE + (1 << 30), 0, 4, 64, 1, 9, None) == UNSUPPORTED
    assert L.rr_reduce(send, FAKE + (1 << 30), 0, 4, 64, 0, 3, None) == UNSUPPORTED  # AVG over int32


def test_broadcast_validation():
    L = rr.lib()
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    for root in (-1, 4):
        assert L.rr_broadcast(FAKE, recv, root, 4, 64, 1, None) == INVALID
    assert L.rr_broadcast(0, recv, 0, 4, 64, 1, None) == INVALID
    # in place at a non-root rank
    bad = rr._ptr_array([FAKE + (1 << 30), FAKE, FAKE + (2 << 30), FAKE + (3 << 30)])
    assert L.rr_broadcast(FAKE, bad, 0, 4, 64, 1, None) == INVALID
    assert L.rr_broadcast(FAKE, recv, 0, 4, 64, 9, None) == UNSUPPORTED


def test_last_error_is_per_call():
    st, msg = ar(p=0)
    assert st == INVALID and msg
    assert ar(n=0)[0] == 0
    assert rr.lib().rr_last_error() == b""


def test_avg_is_float_only():
    """AVG over int32 is refused for every reducing entry point; over the
    float dtypes it passes dtype/op validation (an invalid p then decides)."""
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    assert ar(dt=0, op=3)[0] == UNSUPPORTED
    for algo in (1, 2, 3):
        assert ar(dt=0, op=3, algo=algo, group=2)[0] == UNSUPPORTED
    assert L.rr_reduce_scatter(send, recv, 4, 1024, 0, 3, None) == UNSUPPORTED
    for dt in (1, 2, 3):
        assert ar(p=0, dt=dt, op=3)[0] == INVALID
        assert ar(n=0, dt=dt, op=3)[0] == 0


def test_float16_dtype():
    """float16 is a known dtype of element size 2 (misaligned by 2 bytes is
    fine, by 1 is not)."""
    L = rr.lib()
    assert ar(dt=3, p=0)[0] == INVALID
    assert ar(dt=3, n=0)[0] == 0
    odd = rr._ptr_array([FAKE + 1] + [FAKE + (r << 20) for r in range(1, 4)])
    assert ar(dt=3, send=odd)[0] == INVALID
    out = (ctypes.c_uint64 * 1)()
    assert L.rr_algorithmic_bytes(0, 8, 1000, 3, 0, out) == 0 and out[0] == 2 * 8 * 1000 * 2
    assert rr.workspace_size("ring_staged", 8, 0, 1000, "float16") == 8 * 1000 * 4
    assert rr.workspace_size("ring_staged", 8, 0, 1000, "bfloat16") == 8 * 1000 * 4
    assert rr.workspace_size("ring_staged", 8, 0, 1000, "float32") == 0


def test_scatter_validation():
    L = rr.lib()
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    for root in (-1, 4):
        assert L.rr_scatter(FAKE, recv, root, 4, 64, 1, None) == INVALID
    assert L.rr_scatter(FAKE, recv, 0, 4, 66, 1, None) == INVALID  # p does not divide n
    assert L.rr_scatter(0, recv, 0, 4, 64, 1, None) == INVALID
    assert L.rr_scatter(FAKE, None, 0, 4, 64, 1, None) == INVALID
    assert L.rr_scatter(FAKE, recv, 0, 4, 64, 7, None) == UNSUPPORTED
    assert L.rr_scatter(FAKE, recv, 0, 4, 0, 1, None) == 0
    # a slice output inside the root's buffer at the wrong slot
    bad = rr._ptr_array([FAKE + 16 * 4, FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)])
    assert L.rr_scatter(FAKE, bad, 0, 4, 64, 1, None) == INVALID
    # two outputs overlapping
    bad = rr._ptr_array([FAKE + (1 << 30), FAKE + (1 << 30) + 8, FAKE + (3 << 30), FAKE + (4 << 30)])
    assert L.rr_scatter(FAKE, bad, 0, 4, 64, 1, None) == INVALID


def test_gather_validation():
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    for root in (-1, 4):
        assert L.rr_gather(send, FAKE + (1 << 30), root, 4, 64, 1, None) == INVALID
    assert L.rr_gather(send, FAKE + (1 << 30), 0, 4, 66, 1, None) == INVALID
    assert L.rr_gather(send, 0, 0, 4, 64, 1, None) == INVALID
    assert L.rr_gather(None, FAKE + (1 << 30), 0, 4, 64, 1, None) == INVALID
    assert L.rr_gather(send, FAKE + (1 << 30), 0, 4, 64, 7, None) == UNSUPPORTED
    # the output over rank 1's slice source
    assert L.rr_gather(send, FAKE + (1 << 20), 0, 4, 64, 1, None) == INVALID
    out = (ctypes.c_uint64 * 1)()
    assert L.rr_algorithmic_bytes(5, 4, 64, 1, 0, out) == 0 and out[0] == 2 * 64 * 4
    assert L.rr_algorithmic_bytes(6, 4, 64, 1, 1, out) == 0 and out[0] == 2 * 48 * 4


def hier(flags, p=4, n=1024, dt=2, op=0, group=2, ws=None, wsb=0):
    L = rr.lib()
    send = ptrs(FAKE, p, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), p, 1 << 20)
    return L.rr_all_reduce_hier(send, recv, p, n, dt, op, group, flags, ws, wsb, None)


def test_hier_variant_validation():
    assert hier(8) == INVALID  # unknown flag bit
    assert hier(1 | 4) == UNSUPPORTED  # staged + intra ring
    assert hier(0, group=3) == INVALID
    assert hier(4) == INVALID  # staged without workspace
    assert hier(2, dt=0, op=3) == UNSUPPORTED  # AVG over int32
    for flags in (0, 1, 2, 3, 6):
        assert hier(flags, n=0) == 0
    L = rr.lib()
    assert L.rr_hier_workspace_size(4, 2, 1000, 2, 0) == 0
    assert L.rr_hier_workspace_size(4, 2, 1000, 2, 4) == 2 * 1000 * 4
    assert L.rr_hier_workspace_size(4, 2, 1000, 2, 6) == 2 * 1000 * 2  # bf16 partials on the wire
    assert L.rr_hier_workspace_size(4, 2, 1000, 1, 6) == 2 * 1000 * 4  # float32: rounding is the identity
    assert L.rr_hier_workspace_size(4, 3, 1000, 2, 4) == 0
    assert L.rr_hier_workspace_size(4, 2, 1001, 2, 4) == 2 * 4016
    assert L.rr_hier_workspace_size(4, 2, 1001, 2, 6) == 2 * 2016  # bf16 partials: 2002 bytes, rounded up
    assert L.rr_hier_workspace_size(4, 2, 1000, 2, 8) == 0


def test_bucket_validation():
    L = rr.lib()
    send = ptrs(FAKE, 8, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), 8, 1 << 20)
    counts = (ctypes.c_size_t * 2)(100, 50)
    assert L.rr_all_reduce_bucket(send, recv, counts, -1, 4, 1, 0, None) == INVALID
    assert L.rr_all_reduce_bucket(send, recv, None, 2, 4, 1, 0, None) == INVALID
    assert L.rr_all_reduce_bucket(None, recv, counts, 2, 4, 1, 0, None) == INVALID
    assert L.rr_all_reduce_bucket(send, recv, counts, 2, 4, 0, 3, None) == UNSUPPORTED
    assert L.rr_all_reduce_bucket(send, recv, counts, 0, 4, 1, 0, None) == 0
    # overlapping outputs across tensors
    bad = rr._ptr_array([FAKE + (1 << 30) + r * 16 for r in range(8)])
    assert L.rr_all_reduce_bucket(send, bad, counts, 2, 4, 1, 0, None) == INVALID
    zero = (ctypes.c_size_t * 2)(0, 0)
    assert L.rr_all_reduce_bucket(send, recv, zero, 2, 4, 1, 0, None) == 0


def test_dim1_validation():
    L = rr.lib()
    send = ptrs(FAKE, 4, 1 << 20)
    recv = ptrs(FAKE + (1 << 30), 4, 1 << 20)
    assert L.rr_all_gather_dim1(send, recv, 4, 3, 10, 1, None) == INVALID  # 4 does not divide 10
    assert L.rr_reduce_scatter_dim1(send, recv, 4, 3, 10, 1, 0, None) == INVALID
    assert L.rr_reduce_scatter_dim1(send, recv, 4, 3, 8, 0, 3, None) == UNSUPPORTED
    assert L.rr_all_gather_dim1(send, recv, 4, 0, 8, 1, None) == 0
    # an output over an input
    bad = rr._ptr_array([FAKE + 64, FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)])
    assert L.rr_reduce_scatter_dim1(send, bad, 4, 3, 8, 1, 0, None) == INVALID
    # (the shards are [3, 2]: 24 bytes of float32; an output 8 bytes in overlaps shard 0)
    bad = rr._ptr_array([FAKE + 8, FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)])
    assert L.rr_all_gather_dim1(send, bad, 4, 3, 8, 1, None) == INVALID


def test_noalloc_refusals_before_any_launch():
    """rr_all_reduce_ex_noalloc refuses a workspace need above its fixed
    scratch (RR_NOALLOC_SCRATCH_BYTES = 64 MiB) and the persistent executor,
    and passes invalid arguments on to rr_all_reduce_ex's checks -- all
    before any HIP call."""
    L = rr.lib()
    scratch = 64 << 20
    p, dt_bf16, staged, hier_staged, persistent = 8, 2, 1, 3, 4
    send, recv = ptrs(FAKE, p, 1 << 30), ptrs(FAKE + (64 << 30), p, 1 << 30)
    n = scratch // (p * 4) + 8  # the staged ring's float32 partials: p*n*4 bytes
    assert L.rr_workspace_size(staged, p, 0, n, dt_bf16) > scratch
    assert L.rr_all_reduce_ex_noalloc(send, recv, p, n, dt_bf16, 0, staged, 0, None) == INVALID
    assert b"scratch" in L.rr_last_error()
    # the staged hierarchy: (p/G) partials of n*4 bytes, each rounded up to 16
    n = scratch // 8 + 4
    assert L.rr_all_reduce_ex_noalloc(send, recv, p, n, dt_bf16, 0, hier_staged, 2, None) == INVALID
    assert b"scratch" in L.rr_last_error()
    assert L.rr_all_reduce_ex_noalloc(send, recv, p, 1024, dt_bf16, 0, persistent, 0, None) == UNSUPPORTED
    # invalid arguments reach rr_all_reduce_ex's own checks
    assert L.rr_all_reduce_ex_noalloc(send, recv, 0, 1024, dt_bf16, 0, staged, 0, None) == INVALID
    assert b"p=" in L.rr_last_error()
    assert L.rr_all_reduce_ex_noalloc(send, recv, p, 1024, 9, 0, staged, 0, None) == UNSUPPORTED
