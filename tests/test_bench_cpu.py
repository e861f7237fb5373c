"""CPU checks of bench.py's CPU-baseline helpers (no GPU): the threaded
formula fold computes the oracle's all-reduce (it checks itself against
oracle.all_reduce_fold before timing) and reports its thread count."""

import os

import pytest

import bench
import workloads as W


@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("bfloat16", "max"), ("int32", "sum")])
def test_threaded_formula_fold(dtype, op):
    p, m = 8, 8 * 5000 + 24
    x = W.random_inputs(7, p, m, dtype, kind="full" if dtype == "int32" else "normal")
    r = bench.threaded_formula_fold(x, op, dtype, 0.05)
    assert r["threads"] == len(os.sched_getaffinity(0))
    assert r["unit"] == "GB/s" and r["value"] > 0


def test_gpus_above_one_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
