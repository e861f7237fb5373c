"""The CPU oracle against its pins (no GPU)."""

import pytest

import oracle_pins as P

DTYPES = ("int32", "float32", "bfloat16")
FLOATS = ("float32", "bfloat16")


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example(dtype):
    P.pin_worked_example(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_worked_example_max_min(dtype):
    P.pin_worked_example_max_min(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("p,n", [(1, 7), (2, 33), (3, 100), (4, 4096), (5, 1003), (8, 4099), (8, 8192)])
def test_closed_form(p, n, dtype):
    P.pin_closed_form(p, n, dtype)


@pytest.mark.parametrize("dtype", FLOATS)
def test_ring_order_probe(dtype):
    P.pin_ring_order_probe(dtype)


@pytest.mark.parametrize("dtype", FLOATS)
def test_reduce_order_probe(dtype):
    P.pin_reduce_order_probe(dtype)


@pytest.mark.parametrize("dtype", FLOATS)
def test_hierarchical_probe(dtype):
    P.pin_hier_probe(dtype)


def test_bf16_rounding_hand():
    P.pin_bf16_rounding_hand()


def test_bf16_nan():
    P.pin_bf16_nan()


def test_bf16_ulp_distance():
    P.pin_bf16_ulp_distance()


def test_bf16_vs_torch():
    P.pin_bf16_vs_torch()


def test_int32_wrap():
    P.pin_int32_wrap()


def test_max_min_signed_zero():
    P.pin_max_min_signed_zero()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_int(seed):
    P.pin_bruteforce_int(seed)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_float(seed):
    P.pin_bruteforce_float(seed)


def test_identities():
    P.pin_identities(11)


@pytest.mark.parametrize("p", [1, 2, 3, 4, 5, 8, 16])
def test_schedule_symbolic(p):
    P.pin_schedule_symbolic(p)


def test_hier_vs_flat():
    P.pin_hier_vs_flat(5)


def test_edge_cases():
    P.pin_edge_cases()


def test_fp16_rounding_hand():
    P.pin_fp16_rounding_hand()


def test_fp16_vs_numpy():
    P.pin_fp16_vs_numpy()


def test_fp16_order_probes():
    P.pin_fp16_order_probes()


def test_fp16_sum_rounds_once():
    P.pin_fp16_sum_rounds_once()


def test_avg_worked_example():
    P.pin_avg_worked_example()


@pytest.mark.parametrize("p,n", [(1, 7), (3, 100), (5, 1003), (8, 4099)])
def test_avg_closed_form(p, n):
    P.pin_avg_closed_form(p, n)


def test_avg_division_probes():
    P.pin_avg_division_probes()


@pytest.mark.parametrize("seed", [0, 1])
def test_avg_correctly_rounded(seed):
    P.pin_avg_correctly_rounded(seed)


def test_avg_ring_order_and_int():
    P.pin_avg_ring_order_and_int()


def test_scatter_gather():
    P.pin_scatter_gather()


def test_bucket():
    P.pin_bucket()


def test_all_gather_dim1():
    P.pin_all_gather_dim1()


def test_reduce_scatter_cols():
    P.pin_reduce_scatter_cols()


def test_hier_variants():
    P.pin_hier_variants()


def test_cost_ring():
    P.pin_cost_ring()


def test_cost_hier_example():
    P.pin_cost_hier_example()
