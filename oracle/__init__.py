"""CPU oracle for the collective reductions over p rank buffers.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or helpers with the HIP library; it imports NumPy and the standard
library only.

Sources (web pages; cited by title and section):

* "分布式训练/推理" (llm-from-scratch, chapter 7), section
  "通信原语：rank、world size 和 collective operations": the semantics table of
  broadcast / scatter / gather / reduce / all-gather / reduce-scatter /
  all-reduce, the all-reduce formula y = sum_r x_r, and the worked example
  x_r = [0,1,2,3] + r for p = 4 together with the identity
  all_reduce = reduce_scatter + all_gather.
* "LLM Parallelism 基础", section "Ring AllReduce": the data is cut evenly into
  as many chunks as there are ranks; phase 1 (reduce-scatter) takes N-1 steps
  in which every rank passes one chunk to the next rank on the ring and the
  receiver accumulates it; phase 2 (all-gather) takes N-1 steps in which the
  receiver overwrites; 2(N-1) steps in all; afterwards rank c holds the fully
  reduced chunk c.  Section "MPI Collective Operations": reduce, broadcast,
  and all-reduce having the effect of reduce followed by broadcast.
* "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片", section
  "Source Log: 2026-05-05" (hierarchical AllReduce + SHARP, steps 1-6): reduce
  inside each node, one representative (GPU0) per node, the representatives'
  results combined across nodes, the result broadcast back inside each node.
* "分布式训练/推理", sections on data parallelism (the averaged gradient, the
  flattened gradient bucket) and tensor parallelism (all-gather of [B, d/p]
  outputs along dim 1; the scatter strategy's reduce of partial outputs
  followed by a scatter of output slices).

Readings where the pages are silent (fold order, ring direction, bf16
rounding, max/min tie rule, int32 overflow) are stated in the docstrings of
``collectives`` and ``bf16``.

Parity pins: every public function is pinned by ``tests/test_oracle.py``
against the worked example, closed forms, hand-computed IEEE-754 probes and
brute force; none is "parity unpinned".
"""

from . import bf16, cost, fp16  # noqa: F401
from .collectives import (  # noqa: F401
    ALL_DTYPES,
    ALL_OPS,
    DTYPES,
    OPS,
    all_gather,
    all_gather_dim1,
    all_reduce_bucket,
    all_reduce_fold,
    all_reduce_hier,
    all_reduce_ring,
    broadcast,
    chunk_bounds,
    fold_elements_ring_order,
    gather,
    reduce,
    reduce_scatter_cols,
    reduce_scatter_ring,
    ring_schedule,
    scatter,
    simulate_ring,
)
