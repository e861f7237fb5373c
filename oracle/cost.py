"""Alpha-beta time model of the collectives, as the pages state it (test
infrastructure: only the tests import this module).

* Page "分布式训练/推理", section "从单卡到多卡": one communication costs a
  fixed latency alpha plus its bytes over the link bandwidth.
* Same page, section "Ring all-reduce 的带宽账": a ring reduce-scatter takes
  N-1 rounds in which every device sends S/N bytes, and so does the ring
  all-gather; the all-reduce chains the two.  The page drops the latency; the
  reading taken here charges one alpha per round, each round being one
  message of S/N bytes.
* Page "大模型并行的最小闭环：集合通信、TP、FSDP/ZeRO-3 到权重分片", section
  "总体时间模型": without the hierarchy a node's B*N bytes cross the slow
  links, T = T_slow(B*N); with it the node first combines on the fast links
  and ships only B, T = T_fast(B*N) + T_slow(B).
"""


def message(alpha_s, bytes_per_s, nbytes):
    """Seconds of one message of ``nbytes`` bytes."""
    return alpha_s + nbytes / bytes_per_s


def ring_all_reduce(p, nbytes, alpha_s, bytes_per_s):
    """Reduce-scatter rounds then all-gather rounds, one message of S/p each."""
    t = 0.0
    for _phase in ("reduce-scatter", "all-gather"):
        for _round in range(p - 1):
            t += message(alpha_s, bytes_per_s, nbytes / p)
    return t


def hier_all_reduce(group_size, nbytes, fast, slow):
    """(t_flat, t_hier) for groups of ``group_size`` ranks of ``nbytes`` each;
    ``fast``/``slow`` are (alpha_s, bytes_per_s)."""
    node_bytes = group_size * nbytes
    t_flat = message(*slow, node_bytes)
    t_hier = message(*fast, node_bytes) + message(*slow, nbytes)
    return t_flat, t_hier
