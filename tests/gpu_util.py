"""Helpers for the GPU tests: moving oracle-format arrays to and from the
device, and choosing sampled positions for full-size comparisons."""

import numpy as np

from oracle import collectives as C


def torch_dtype(dtype):
    import torch

    return {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16,
            "float16": torch.float16}[dtype]


def to_dev(arr, dtype, device="cuda"):
    """(…) numpy storage array -> device tensor of the matching torch dtype."""
    import torch

    arr = np.ascontiguousarray(arr)
    if dtype in ("bfloat16", "float16"):
        t = torch.from_numpy(arr.view(np.int16).copy()).view(torch_dtype(dtype))
    else:
        t = torch.from_numpy(arr.copy())
    return t.to(device)


def to_host(t, dtype):
    """Device tensor -> numpy storage array (16-bit floats as uint16 bit patterns)."""
    import torch

    t = t.detach().cpu().contiguous()
    if dtype in ("bfloat16", "float16"):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view({2: np.uint16, 4: np.uint32, 8: np.uint64}[a.itemsize])


def assert_bitwise(got, want, what=""):
    g, w = bits(got), bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.nonzero(g != w)
    if bad[0].size:
        idx = tuple(b[:8] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} mismatches, first at {idx}: got {g[idx]} want {w[idx]}")


def sample_positions(n, p, count, seed):
    """Chunk edges, the ends of the vector and ``count`` random positions."""
    rng = np.random.default_rng(seed)
    b = C.chunk_bounds(n, p)
    edges = []
    for c in range(p):
        for e in (b[c], b[c] + 1, b[c] + 2, b[c + 1] - 1, b[c + 1] - 2, b[c + 1] - 3):
            if b[c] <= e < b[c + 1]:
                edges.append(e)
    pos = np.concatenate([np.array(edges, dtype=np.int64), rng.integers(0, n, size=count, dtype=np.int64),
                          np.array([0, n - 1], dtype=np.int64)])
    return np.unique(pos)


def chunk_of(positions, n, p):
    b = np.array(C.chunk_bounds(n, p), dtype=np.int64)
    return np.searchsorted(b[1:], positions, side="right")


def ring_fold_blocks(x, op, dtype, block=1 << 20):
    """The oracle's ring-order fold of EVERY element of (p, n) inputs, in
    blocks of at most ``block`` elements that each lie inside one chunk (so
    that host memory stays bounded at full size).  Yields (lo, hi, result)."""
    p, n = x.shape
    b = C.chunk_bounds(n, p)
    for c in range(p):
        for lo in range(b[c], b[c + 1], block):
            hi = min(lo + block, b[c + 1])
            yield lo, hi, C.fold_elements_ring_order(x[:, lo:hi], np.full(hi - lo, c), op, dtype)
