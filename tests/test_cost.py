"""The C cost model of librr.so (host only, no GPU) against the oracle's
statement of the pages' time model, and its argument checks."""

import numpy as np
import pytest

import collective_communication_reduction_way_amd as rr
from oracle import cost as K


def close(a, b):
    return abs(a - b) <= 1e-12 * max(abs(a), abs(b), 1e-300)


def test_ring_matches_oracle():
    rng = np.random.default_rng(1)
    for _ in range(500):
        p = int(rng.integers(1, 65))
        nbytes = float(rng.uniform(0, 1e10))
        alpha = float(rng.uniform(0, 1e-4))
        bw = float(10 ** rng.uniform(8, 13))
        assert close(rr.cost_ring_all_reduce(p, nbytes, alpha, bw), K.ring_all_reduce(p, nbytes, alpha, bw))


def test_hier_matches_oracle():
    rng = np.random.default_rng(2)
    for _ in range(500):
        G = int(rng.integers(1, 65))
        nbytes = float(rng.uniform(0, 1e9))
        fast = (float(rng.uniform(0, 1e-5)), float(10 ** rng.uniform(10, 13)))
        slow = (float(rng.uniform(0, 1e-4)), float(10 ** rng.uniform(8, 11)))
        tf, th, use = rr.cost_hier_all_reduce(G, nbytes, fast, slow)
        wf, wh = K.hier_all_reduce(G, nbytes, fast, slow)
        assert close(tf, wf) and close(th, wh) and use == (wh < wf)


def test_page_example_through_the_library():
    tf, th, use = rr.cost_hier_all_reduce(4, 8e6, (0.0, 1.8e12), (0.0, 0.05e12))
    assert close(tf, 640e-6) and close(th, 32e6 / 1.8e12 + 160e-6) and use


@pytest.mark.parametrize("args", [(0, 1.0, 0.0, 1.0), (65, 1.0, 0.0, 1.0), (4, -1.0, 0.0, 1.0), (4, 1.0, -1.0, 1.0),
                                  (4, 1.0, 0.0, 0.0)])
def test_ring_rejects(args):
    with pytest.raises(rr.RRError):
        rr.cost_ring_all_reduce(*args)


def test_hier_rejects():
    with pytest.raises(rr.RRError):
        rr.cost_hier_all_reduce(0, 1.0, (0.0, 1.0), (0.0, 1.0))
    with pytest.raises(rr.RRError):
        rr.cost_hier_all_reduce(4, 1.0, (0.0, 0.0), (0.0, 1.0))
