"""Seeded synthetic workloads for the collective reductions.

Shared by the tests and ``bench.py``; holds no arithmetic of the collectives
themselves (only random draws and the storage encoding of the inputs).  Rank
r of a workload draws its buffer from ``numpy.random.default_rng([seed, r])``,
one independent stream per (workload, rank) -- the per-rank seeding practice
of page "分布式训练/推理" (section on seeds in the data-loading part).

bfloat16 inputs are drawn in float32 and encoded to bf16 bit patterns with
torch's CPU conversion (round to nearest even), float16 inputs with numpy's
float16 conversion (the same rounding); the arrays returned here use the
storage types of the oracle: int32, float32, and uint16 bit patterns for
bfloat16 and float16.

Workloads (sizes in elements per rank):
  ar_int32_p4_n4096         sum all-reduce, p=4, 4,096 int32, uniform in
                            [-2^20, 2^20] (ring schedule of 6 steps)
  ar_fp32_p8_8MiB           sum all-reduce, p=8, 2,097,152 fp32 (8 MiB per
                            rank), standard normal
  hier_bf16_p8g4_8MiB       hierarchical sum all-reduce, p=8 as 2 groups of 4,
                            4,194,304 bf16 (8 MiB per rank), standard normal
  zero_bucket_fp32_p8       gradient bucket: p=8, 25,165,824 fp32 per rank,
                            N(0, sigma=1e-3); reduce-scatter to n/p shards,
                            all-gather, and all-reduce with sum, max and min
  tp_rowparallel_bf16_p8    row-parallel partial outputs: p=8 partials of
                            shape (8, 2048, 4096) bf16, N(0, sigma=1/sqrt(8))

Bucket of gradients (``BUCKETS``): the parameter tensors of one transformer
block laid out as a DDP gradient bucket, tensor by tensor in parameter order:
  gpt2_block_fp32_p8        p=8, d=768 (GPT-2 small): qkv weight 768x2304 and
                            bias, attention projection 768x768 and bias, two
                            layer-norm weight/bias pairs, MLP 768x3072 and
                            3072x768 with biases -- 12 tensors, 7,087,872 fp32
                            per rank (27 MiB), N(0, sigma=1e-3)
"""

import math

import numpy as np

STORAGE = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16, "float16": np.uint16}

WORKLOADS = {
    "ar_int32_p4_n4096": dict(
        coll="all_reduce", algo="ring", p=4, n=4096, dtype="int32", dist="uniform_int", limit=2 ** 20, seed=1,
        ops=("sum",)),
    "ar_fp32_p8_8MiB": dict(
        coll="all_reduce", algo="ring", p=8, n=2097152, dtype="float32", dist="normal", sigma=1.0, seed=2,
        ops=("sum",)),
    "hier_bf16_p8g4_8MiB": dict(
        coll="all_reduce", algo="hier", group=4, p=8, n=4194304, dtype="bfloat16", dist="normal", sigma=1.0,
        seed=3, ops=("sum",)),
    "zero_bucket_fp32_p8": dict(
        coll="rs_ag", algo="ring", p=8, n=25165824, dtype="float32", dist="normal", sigma=1e-3, seed=4,
        ops=("sum", "max", "min")),
    "tp_rowparallel_bf16_p8": dict(
        coll="all_reduce", algo="ring", p=8, n=8 * 2048 * 4096, shape=(8, 2048, 4096), dtype="bfloat16",
        dist="normal", sigma=1.0 / math.sqrt(8.0), seed=5, ops=("sum",)),
}


def _gpt2_block(d):
    return [d * 3 * d, 3 * d, d * d, d, d, d, d * 4 * d, 4 * d, 4 * d * d, d, d, d]


BUCKETS = {
    "gpt2_block_fp32_p8": dict(p=8, sizes=_gpt2_block(768), dtype="float32", sigma=1e-3, seed=6),
}


def bucket_inputs(name):
    """The bucket's tensors as a list of (p, n_t) arrays (rows = ranks)."""
    spec = BUCKETS[name]
    out = []
    for t, n in enumerate(spec["sizes"]):
        rows = []
        for r in range(spec["p"]):
            rng = np.random.default_rng([spec["seed"], t, r])
            x = rng.standard_normal(n, dtype=np.float32) * np.float32(spec["sigma"])
            rows.append(x)
        out.append(np.stack(rows))
    return out


def _bf16_bits(f32):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rank_input(spec, r, count=None):
    """Rank r's buffer (first ``count`` elements, default all n) in storage type."""
    n = spec["n"] if count is None else int(count)
    rng = np.random.default_rng([spec["seed"], r])
    if spec["dist"] == "uniform_int":
        lim = spec["limit"]
        return rng.integers(-lim, lim, size=n, endpoint=True, dtype=np.int64).astype(np.int32)
    x = rng.standard_normal(n, dtype=np.float32)
    if spec["sigma"] != 1.0:
        x *= np.float32(spec["sigma"])
    if spec["dtype"] == "float32":
        return x
    return _bf16_bits(x)


def make_inputs(name, count=None):
    """The (p, n) input array of a named workload (rows = ranks)."""
    spec = WORKLOADS[name]
    return np.stack([rank_input(spec, r, count) for r in range(spec["p"])])


def _f16_bits(f32):
    return np.ascontiguousarray(f32, dtype=np.float32).astype(np.float16).view(np.uint16).copy()


def random_inputs(seed, p, n, dtype, kind="normal"):
    """Generic seeded inputs for parity sweeps: normal values (fp32 / bf16 /
    fp16), every finite float16 bit pattern equally likely ("fp16_patterns",
    float16 only: subnormals to 65504, so sums meet every rounding case and
    overflow), or int32 over the full range ("full") or in [-2^20, 2^20]
    ("small")."""
    rng = np.random.default_rng([seed, p, n])
    if dtype == "int32":
        if kind == "full":
            return rng.integers(-(2 ** 31), 2 ** 31, size=(p, n), dtype=np.int64).astype(np.int32)
        return rng.integers(-(2 ** 20), 2 ** 20, size=(p, n), endpoint=True, dtype=np.int64).astype(np.int32)
    if kind == "fp16_patterns":
        assert dtype == "float16"
        mag = rng.integers(0, 0x7C00, size=(p, n), dtype=np.int64)
        sign = rng.integers(0, 2, size=(p, n), dtype=np.int64) << 15
        return (mag | sign).astype(np.uint16)
    x = rng.standard_normal((p, n), dtype=np.float32)
    if dtype == "float32":
        return x
    if dtype == "float16":
        return _f16_bits(x).reshape(p, n)
    return _bf16_bits(x).reshape(p, n)
