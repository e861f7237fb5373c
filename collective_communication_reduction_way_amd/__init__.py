"""rr -- collective reductions over p virtual ranks resident in one MI355X's HBM.

A thin ctypes binding over the C ABI of ``librr.so`` (declared in
``include/rr.h``).  It only marshals arguments: tensors become device
pointers, the stream defaults to torch's current stream, and every step of
every collective runs in the library's HIP kernels.  There is no fallback: if
``librr.so`` is missing or cannot be loaded, every call raises.

Rank buffers are given either as a list of p tensors or as one 2-D tensor
whose rows are the ranks.  All tensors must be contiguous, on one device and
of one dtype (int32, float32, bfloat16 or float16).  Ops: "sum", "max",
"min" and, for the float dtypes, "avg" (the sum divided by p).

Semantics (pages cited by title and section):
  page "分布式训练/推理", section "通信原语：rank、world size 和 collective
  operations" -- broadcast, reduce, all-gather, reduce-scatter, all-reduce;
  page "LLM Parallelism 基础", section "Ring AllReduce" -- the ring schedule
  whose reduce-scatter order the all-reduce and reduce-scatter follow;
  page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片", section
  "Source Log: 2026-05-05" -- the hierarchical all-reduce.
"""

import ctypes
import os

__all__ = [
    "RRError",
    "all_reduce",
    "reduce_scatter",
    "all_gather",
    "reduce",
    "broadcast",
    "scatter",
    "gather",
    "all_reduce_bucket",
    "all_gather_dim1",
    "reduce_scatter_dim1",
    "all_reduce_hier",
    "hier_workspace_size",
    "cost_ring_all_reduce",
    "cost_hier_all_reduce",
    "workspace_size",
    "ring_schedule",
    "chunk_bounds",
    "algorithmic_bytes",
    "ring_bytes_per_rank",
    "hier_traffic",
    "library_path",
    "lib",
    "version",
    "barrier_timeouts",
    "ring_exec_failures",
    "reload_tuning",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librr.so")

DTYPES = {"int32": 0, "float32": 1, "bfloat16": 2, "float16": 3}
OPS = {"sum": 0, "max": 1, "min": 2, "avg": 3}
ALGOS = {"ring": 0, "ring_staged": 1, "hier": 2, "hier_staged": 3, "ring_persistent": 4}
COLLS = {"all_reduce": 0, "reduce_scatter": 1, "all_gather": 2, "reduce": 3, "broadcast": 4, "scatter": 5,
         "gather": 6}
MAX_RANKS = 64
HIER_INTRA_RING, HIER_WIRE_ROUND, HIER_STAGED = 1, 2, 4


class _Link(ctypes.Structure):
    _fields_ = [("alpha_s", ctypes.c_double), ("bytes_per_s", ctypes.c_double)]

_lib = None


class RRError(RuntimeError):
    """A librr call returned a non-success status."""

    def __init__(self, status, func, message):
        self.status = status
        super().__init__(f"{func}: status {status} ({message})")


def library_path():
    return _LIB_PATH


def lib():
    """Load librr.so once (after torch, so that the library binds to the HIP
    runtime torch has already loaded) and declare every signature."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (loads torch's HIP runtime first)

    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -m collective_communication_reduction_way_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(ctypes.c_void_p)
    I = ctypes.c_int
    S = ctypes.c_size_t
    U64P = ctypes.POINTER(ctypes.c_uint64)
    IP = ctypes.POINTER(ctypes.c_int)
    sig = {
        "rr_all_reduce": (I, [PP, PP, I, S, I, I, P]),
        "rr_all_reduce_ex": (I, [PP, PP, I, S, I, I, I, I, P, S, P]),
        "rr_all_reduce_ex_noalloc": (I, [PP, PP, I, S, I, I, I, I, P]),
        "rr_reduce_scatter": (I, [PP, PP, I, S, I, I, P]),
        "rr_all_gather": (I, [PP, PP, I, S, I, P]),
        "rr_reduce": (I, [PP, P, I, I, S, I, I, P]),
        "rr_broadcast": (I, [P, PP, I, I, S, I, P]),
        "rr_scatter": (I, [P, PP, I, I, S, I, P]),
        "rr_gather": (I, [PP, P, I, I, S, I, P]),
        "rr_all_reduce_bucket": (I, [PP, PP, ctypes.POINTER(ctypes.c_size_t), I, I, I, I, P]),
        "rr_all_gather_dim1": (I, [PP, PP, I, S, S, I, P]),
        "rr_reduce_scatter_dim1": (I, [PP, PP, I, S, S, I, I, P]),
        "rr_all_reduce_hier": (I, [PP, PP, I, S, I, I, I, I, P, S, P]),
        "rr_hier_workspace_size": (S, [I, I, S, I, I]),
        "rr_cost_ring_all_reduce": (I, [I, ctypes.c_double, _Link, ctypes.POINTER(ctypes.c_double)]),
        "rr_cost_hier_all_reduce": (I, [I, ctypes.c_double, _Link, _Link, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double), IP]),
        "rr_workspace_size": (S, [I, I, I, S, I]),
        "rr_ring_schedule": (I, [I, IP, IP, IP, IP, IP, I]),
        "rr_chunk_bounds": (I, [I, S, ctypes.POINTER(ctypes.c_size_t)]),
        "rr_algorithmic_bytes": (I, [I, I, S, I, I, U64P]),
        "rr_ring_bytes_per_rank": (I, [I, S, I, U64P, U64P]),
        "rr_hier_traffic": (I, [I, I, ctypes.c_uint64, U64P, U64P, U64P]),
        "rr_status_string": (ctypes.c_char_p, [I]),
        "rr_last_error": (ctypes.c_char_p, []),
        "rr_barrier_timeouts": (I, [I, U64P]),
        "rr_ring_exec_failures": (I, [I, U64P]),
        "rr_version": (ctypes.c_char_p, []),
        "rr_reload_tuning": (None, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def barrier_timeouts(device=None):
    """How often a fused fold's soft phase barrier on `device` (default: the
    current device) ended by timeout since the library was loaded.  The
    barrier only shapes HBM traffic, so this counts lost throughput, never
    wrong results.  Synchronizes the device."""
    import torch

    dev = torch.cuda.current_device() if device is None else int(device)
    out = ctypes.c_uint64(0)
    _check(lib().rr_barrier_timeouts(dev, ctypes.byref(out)), "rr_barrier_timeouts")
    return int(out.value)


def ring_exec_failures(device=None):
    """How many launches of the persistent ring executor (algo
    "ring_persistent") on `device` stopped on a timed-out wait since the
    library was loaded (their outputs are incomplete).  Synchronizes the
    device."""
    import torch

    dev = torch.cuda.current_device() if device is None else int(device)
    out = ctypes.c_uint64(0)
    _check(lib().rr_ring_exec_failures(dev, ctypes.byref(out)), "rr_ring_exec_failures")
    return int(out.value)


def version():
    return lib().rr_version().decode()


def reload_tuning():
    """Read the RR_* tuning variables of the environment again (the library
    reads them once, at its first call); later calls use the new values."""
    lib().rr_reload_tuning()


def _check(status, func):
    if status != 0:
        msg = lib().rr_last_error().decode() or lib().rr_status_string(status).decode()
        raise RRError(status, func, msg)


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, v in enumerate(ptrs):
        arr[i] = v
    return arr


def _dtype_name(dtype):
    import torch

    m = {torch.int32: "int32", torch.float32: "float32", torch.bfloat16: "bfloat16", torch.float16: "float16"}
    if dtype not in m:
        raise TypeError(f"unsupported dtype {dtype}; use int32, float32, bfloat16 or float16")
    return m[dtype]


def _dtype_code(t):
    return DTYPES[_dtype_name(t.dtype)]


def _ranks(bufs, what):
    """A list of tensors or a 2-D tensor (rows = ranks) -> list of tensors."""
    import torch

    if isinstance(bufs, torch.Tensor):
        if bufs.dim() != 2:
            raise ValueError(f"{what}: a tensor of rank buffers must be 2-D (p, n)")
        bufs = list(bufs.unbind(0))
    bufs = list(bufs)
    if not bufs:
        raise ValueError(f"{what}: no rank buffers")
    d, dt = bufs[0].device, bufs[0].dtype
    for t in bufs:
        if not t.is_contiguous():
            raise ValueError(f"{what}: rank buffers must be contiguous")
        if t.device != d or t.dtype != dt:
            raise ValueError(f"{what}: rank buffers must share device and dtype")
    return bufs


def _stream(t, stream):
    import torch

    if stream is None:
        if t.device.type != "cuda":
            raise ValueError("rank buffers must be GPU tensors")
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call_workspace(nbytes, t, stream):
    """A device workspace for one call, allocated with torch on the current
    stream.  When the kernels go to another stream, the tensor is marked as
    used by that stream, so that torch's caching allocator does not hand the
    block to new work on the current stream while those kernels still write
    it (the tensor is freed as soon as the call returns)."""
    import torch

    ws = torch.empty(nbytes, dtype=torch.uint8, device=t.device)
    if stream is not None:
        if isinstance(stream, int):
            stream = torch.cuda.ExternalStream(stream, device=t.device)
        ws.record_stream(stream)
    return ws


def _op(op):
    if op not in OPS:
        raise ValueError(f"unknown op {op!r}; use one of {sorted(OPS)}")
    return OPS[op]


def all_reduce(ins, outs=None, op="sum", algo="ring", group_size=0, workspace=None, stream=None):
    """Every rank's output becomes the reduction of all p inputs.

    outs=None reduces in place.  algo: "ring" (one fused pass in ring order),
    "ring_staged" (the ring schedule step by step, one launch per step),
    "ring_persistent" (the ring schedule in one persistent kernel), "hier" /
    "hier_staged" (groups of ``group_size`` consecutive ranks).  The staged algorithms may
    need a device workspace of ``workspace_size(...)`` bytes (a uint8 tensor);
    when it is not given, one is allocated with torch for the call.
    """
    ins = _ranks(ins, "all_reduce inputs")
    outs = ins if outs is None else _ranks(outs, "all_reduce outputs")
    p, n = len(ins), ins[0].numel()
    if len(outs) != p or any(o.numel() != n for o in outs) or any(o.dtype != ins[0].dtype for o in outs):
        raise ValueError("all_reduce: outputs must match the inputs in count, length and dtype")
    for t in ins[1:]:
        if t.numel() != n:
            raise ValueError("all_reduce: rank buffers must have equal length")
    if algo not in ALGOS:
        raise ValueError(f"unknown algo {algo!r}; use one of {sorted(ALGOS)}")
    dt = _dtype_code(ins[0])
    need = workspace_size(algo, p, group_size, n, ins[0].dtype)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = _call_workspace(need, ins[0], stream)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    L = lib()
    st = L.rr_all_reduce_ex(_ptr_array([t.data_ptr() for t in ins]), _ptr_array([t.data_ptr() for t in outs]),
                            p, n, dt, _op(op), ALGOS[algo], int(group_size), ws_ptr, ws_bytes,
                            _stream(ins[0], stream))
    _check(st, "rr_all_reduce_ex")
    return outs


def reduce_scatter(ins, outs, op="sum", stream=None):
    """Rank c's output (n/p elements) becomes chunk c of the reduction."""
    ins = _ranks(ins, "reduce_scatter inputs")
    outs = _ranks(outs, "reduce_scatter outputs")
    p, n = len(ins), ins[0].numel()
    if len(outs) != p or any(o.numel() * p != n for o in outs):
        raise ValueError("reduce_scatter: need p outputs of n/p elements")
    L = lib()
    st = L.rr_reduce_scatter(_ptr_array([t.data_ptr() for t in ins]), _ptr_array([t.data_ptr() for t in outs]),
                             p, n, _dtype_code(ins[0]), _op(op), _stream(ins[0], stream))
    _check(st, "rr_reduce_scatter")
    return outs


def all_gather(ins, outs, stream=None):
    """Every rank's output (n elements) becomes the concatenation of the p shards."""
    ins = _ranks(ins, "all_gather inputs")
    outs = _ranks(outs, "all_gather outputs")
    p, n = len(ins), outs[0].numel()
    if len(outs) != p or any(i.numel() * p != n for i in ins):
        raise ValueError("all_gather: need p shards of n/p elements and p outputs of n")
    L = lib()
    st = L.rr_all_gather(_ptr_array([t.data_ptr() for t in ins]), _ptr_array([t.data_ptr() for t in outs]),
                         p, n, _dtype_code(ins[0]), _stream(ins[0], stream))
    _check(st, "rr_all_gather")
    return outs


def reduce(ins, out, root=0, op="sum", stream=None):
    """The root's output becomes the reduction of all p inputs (ascending order)."""
    ins = _ranks(ins, "reduce inputs")
    p, n = len(ins), ins[0].numel()
    if out.numel() != n or out.dtype != ins[0].dtype or not out.is_contiguous():
        raise ValueError("reduce: output must be contiguous with the inputs' length and dtype")
    L = lib()
    st = L.rr_reduce(_ptr_array([t.data_ptr() for t in ins]), out.data_ptr(), int(root), p, n,
                     _dtype_code(ins[0]), _op(op), _stream(ins[0], stream))
    _check(st, "rr_reduce")
    return out


def broadcast(x, outs, root=0, stream=None):
    """Every rank's output becomes a copy of the root's buffer ``x``."""
    outs = _ranks(outs, "broadcast outputs")
    p, n = len(outs), x.numel()
    if any(o.numel() != n or o.dtype != x.dtype for o in outs) or not x.is_contiguous():
        raise ValueError("broadcast: outputs must match the root buffer")
    L = lib()
    st = L.rr_broadcast(x.data_ptr(), _ptr_array([t.data_ptr() for t in outs]), int(root), p, n,
                        _dtype_code(x), _stream(x, stream))
    _check(st, "rr_broadcast")
    return outs


def scatter(x, outs, root=0, stream=None):
    """Rank c's output (n/p elements) becomes slice c of the root's buffer ``x``."""
    outs = _ranks(outs, "scatter outputs")
    p, n = len(outs), x.numel()
    if any(o.numel() * p != n or o.dtype != x.dtype for o in outs) or not x.is_contiguous():
        raise ValueError("scatter: need p outputs of n/p elements of the root buffer's dtype")
    L = lib()
    st = L.rr_scatter(x.data_ptr(), _ptr_array([t.data_ptr() for t in outs]), int(root), p, n, _dtype_code(x),
                      _stream(x, stream))
    _check(st, "rr_scatter")
    return outs


def gather(ins, out, root=0, stream=None):
    """The root's output ``out`` (n elements) becomes the p slices in rank order."""
    ins = _ranks(ins, "gather inputs")
    p, n = len(ins), out.numel()
    if any(i.numel() * p != n or i.dtype != out.dtype for i in ins) or not out.is_contiguous():
        raise ValueError("gather: need p slices of n/p elements of the output's dtype")
    L = lib()
    st = L.rr_gather(_ptr_array([t.data_ptr() for t in ins]), out.data_ptr(), int(root), p, n, _dtype_code(out),
                     _stream(out, stream))
    _check(st, "rr_gather")
    return out


def all_reduce_bucket(tensors, outs=None, op="sum", stream=None):
    """All-reduce a bucket of tensors as if they were laid end to end.

    ``tensors[t]`` holds tensor t of every rank (a list of p tensors or a 2-D
    (p, n_t) tensor); ``outs`` has the same structure (None = in place).  The
    result is bitwise that of ``all_reduce`` on the concatenated bucket.
    """
    tensors = [_ranks(t, f"all_reduce_bucket tensor {i}") for i, t in enumerate(tensors)]
    outs = tensors if outs is None else [_ranks(t, f"all_reduce_bucket output {i}") for i, t in enumerate(outs)]
    if not tensors:
        return outs
    p = len(tensors[0])
    dt = tensors[0][0].dtype
    if len(outs) != len(tensors):
        raise ValueError("all_reduce_bucket: outputs must match the tensors")
    send, recv, counts = [], [], []
    for i, (ti, to) in enumerate(zip(tensors, outs)):
        if len(ti) != p or len(to) != p:
            raise ValueError(f"all_reduce_bucket: tensor {i} needs {p} rank buffers")
        n = ti[0].numel()
        if any(x.numel() != n or x.dtype != dt for x in list(ti) + list(to)):
            raise ValueError(f"all_reduce_bucket: tensor {i}: rank buffers and outputs need equal length and dtype")
        counts.append(n)
        send += [x.data_ptr() for x in ti]
        recv += [x.data_ptr() for x in to]
    cnt = (ctypes.c_size_t * len(counts))(*counts)
    L = lib()
    st = L.rr_all_reduce_bucket(_ptr_array(send), _ptr_array(recv), cnt, len(counts), p,
                                DTYPES[_dtype_name(dt)], _op(op), _stream(tensors[0][0], stream))
    _check(st, "rr_all_reduce_bucket")
    return outs


def _mats(bufs, what):
    """A list of p contiguous matrices or a 3-D (p, rows, cols) tensor."""
    import torch

    if isinstance(bufs, torch.Tensor):
        if bufs.dim() != 3:
            raise ValueError(f"{what}: a tensor of rank matrices must be 3-D (p, rows, cols)")
        bufs = list(bufs.unbind(0))
    bufs = list(bufs)
    for t in bufs:
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{what}: rank matrices must be contiguous 2-D tensors")
    return bufs


def all_gather_dim1(shards, outs, stream=None):
    """Every rank's [rows, p*w] output becomes the concatenation along dim 1 of
    the p [rows, w] shards."""
    shards = _mats(shards, "all_gather_dim1 shards")
    outs = _mats(outs, "all_gather_dim1 outputs")
    p = len(shards)
    rows, w = shards[0].shape
    if len(outs) != p or any(o.shape != (rows, p * w) for o in outs) or any(s.shape != (rows, w) for s in shards):
        raise ValueError("all_gather_dim1: need p shards [rows, w] and p outputs [rows, p*w]")
    L = lib()
    st = L.rr_all_gather_dim1(_ptr_array([t.data_ptr() for t in shards]), _ptr_array([t.data_ptr() for t in outs]),
                              p, rows, p * w, _dtype_code(shards[0]), _stream(shards[0], stream))
    _check(st, "rr_all_gather_dim1")
    return outs


def reduce_scatter_dim1(ins, outs, op="sum", stream=None):
    """Rank c's [rows, cols/p] output becomes feature slice c of the reduction
    of the p [rows, cols] inputs (ring order of chunk c)."""
    ins = _mats(ins, "reduce_scatter_dim1 inputs")
    outs = _mats(outs, "reduce_scatter_dim1 outputs")
    p = len(ins)
    rows, cols = ins[0].shape
    if cols % p or len(outs) != p or any(o.shape != (rows, cols // p) for o in outs) or any(
            i.shape != (rows, cols) for i in ins):
        raise ValueError("reduce_scatter_dim1: need p inputs [rows, cols] and p outputs [rows, cols/p]")
    L = lib()
    st = L.rr_reduce_scatter_dim1(_ptr_array([t.data_ptr() for t in ins]), _ptr_array([t.data_ptr() for t in outs]),
                                  p, rows, cols, _dtype_code(ins[0]), _op(op), _stream(ins[0], stream))
    _check(st, "rr_reduce_scatter_dim1")
    return outs


def _hier_flags(intra, wire_round, staged):
    if intra not in ("reduce", "ring"):
        raise ValueError(f"unknown intra-group step {intra!r}; use 'reduce' or 'ring'")
    return (HIER_INTRA_RING if intra == "ring" else 0) | (HIER_WIRE_ROUND if wire_round else 0) | (
        HIER_STAGED if staged else 0)


def all_reduce_hier(ins, outs=None, op="sum", group_size=1, intra="reduce", wire_round=False, staged=False,
                    workspace=None, stream=None):
    """Hierarchical all-reduce over groups of ``group_size`` consecutive ranks.

    intra="ring" forms each group's partial by a ring all-reduce inside the
    group; wire_round=True rounds every group partial to the storage type
    before the cross-group fold; staged=True runs the steps one by one
    through a workspace (allocated with torch when not given).
    """
    ins = _ranks(ins, "all_reduce_hier inputs")
    outs = ins if outs is None else _ranks(outs, "all_reduce_hier outputs")
    p, n = len(ins), ins[0].numel()
    if len(outs) != p or any(o.numel() != n or o.dtype != ins[0].dtype for o in outs):
        raise ValueError("all_reduce_hier: outputs must match the inputs in count, length and dtype")
    flags = _hier_flags(intra, wire_round, staged)
    need = hier_workspace_size(p, group_size, n, ins[0].dtype, intra, wire_round, staged)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = _call_workspace(need, ins[0], stream)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib().rr_all_reduce_hier(_ptr_array([t.data_ptr() for t in ins]), _ptr_array([t.data_ptr() for t in outs]),
                                  p, n, _dtype_code(ins[0]), _op(op), int(group_size), flags, ws_ptr, ws_bytes,
                                  _stream(ins[0], stream))
    _check(st, "rr_all_reduce_hier")
    return outs


def hier_workspace_size(p, group_size, n, dtype, intra="reduce", wire_round=False, staged=False):
    """Bytes of workspace rr_all_reduce_hier needs (0 unless staged)."""
    import torch

    if isinstance(dtype, torch.dtype):
        dtype = _dtype_name(dtype)
    return int(lib().rr_hier_workspace_size(int(p), int(group_size), int(n), DTYPES[dtype],
                                            _hier_flags(intra, wire_round, staged)))


def cost_ring_all_reduce(p, nbytes, alpha_s, bytes_per_s):
    """Seconds the alpha-beta model gives a ring all-reduce of ``nbytes`` per rank."""
    out = ctypes.c_double()
    _check(lib().rr_cost_ring_all_reduce(int(p), float(nbytes), _Link(alpha_s, bytes_per_s), ctypes.byref(out)),
           "rr_cost_ring_all_reduce")
    return out.value


def cost_hier_all_reduce(group_size, nbytes, fast, slow):
    """(t_flat, t_hier, use_hier) of the hierarchy's time model; ``fast`` and
    ``slow`` are (alpha_s, bytes_per_s) pairs."""
    tf, th, use = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    _check(lib().rr_cost_hier_all_reduce(int(group_size), float(nbytes), _Link(*fast), _Link(*slow),
                                         ctypes.byref(tf), ctypes.byref(th), ctypes.byref(use)),
           "rr_cost_hier_all_reduce")
    return tf.value, th.value, bool(use.value)


def workspace_size(algo, p, group_size, n, dtype):
    """Bytes of workspace rr_all_reduce_ex needs (0 for the fused algorithms)."""
    import torch

    if isinstance(dtype, torch.dtype):
        dtype = _dtype_name(dtype)
    return int(lib().rr_workspace_size(ALGOS[algo], int(p), int(group_size), int(n), DTYPES[dtype]))


# ---------------------------------------------------------------------------
# Host-only planning helpers (no GPU needed).

def ring_schedule(p):
    """The ring's transfers as (phase, step, src, dst, chunk) tuples; phase 0 is
    reduce-scatter (the receiver accumulates), phase 1 all-gather."""
    L = lib()
    total = L.rr_ring_schedule(int(p), None, None, None, None, None, 0)
    if total < 0:
        raise ValueError(f"p={p} out of range")
    arrs = [(ctypes.c_int * max(1, total))() for _ in range(5)]
    L.rr_ring_schedule(int(p), *arrs, total)
    return [tuple(a[i] for a in arrs) for i in range(total)]


def chunk_bounds(p, n):
    b = (ctypes.c_size_t * (int(p) + 1))()
    _check(lib().rr_chunk_bounds(int(p), int(n), b), "rr_chunk_bounds")
    return list(b)


def algorithmic_bytes(coll, p, n, dtype, in_place=False):
    out = ctypes.c_uint64()
    _check(lib().rr_algorithmic_bytes(COLLS[coll], int(p), int(n), DTYPES[dtype], int(bool(in_place)),
                                      ctypes.byref(out)), "rr_algorithmic_bytes")
    return out.value


def ring_bytes_per_rank(p, n, dtype):
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().rr_ring_bytes_per_rank(int(p), int(n), DTYPES[dtype], ctypes.byref(a), ctypes.byref(b)),
           "rr_ring_bytes_per_rank")
    return a.value, b.value


def hier_traffic(p, group_size, bytes_per_rank):
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().rr_hier_traffic(int(p), int(group_size), int(bytes_per_rank), ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)), "rr_hier_traffic")
    return {"intra_per_group": a.value, "cross_per_group_flat": b.value, "cross_per_group_hier": c.value}
