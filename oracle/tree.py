"""Fixed combine schedules over leaves, chunks and splits (oracle side).

[IsoExec] "Parallelism-invariant kernels" (and [NovaSky] "Making kernels
parallelism-invariant"): K is divided into contiguous leaves whose FP32
partials are combined by a binary schedule that the contract fixes, with a
fixed rank-to-leaf mapping. [RLK] section 6 (module 06) uses a fixed
balanced tree for TP 1/2/4/8. [RLK] section 2 shows that the same four
values summed as ((a+b)+c)+d and as (a+b)+(c+d) can round differently.

Reading taken: "balanced" is recursive halving with the left half holding the
first ceil(n/2) items; for a power of two this pairs adjacent items first,
so every aligned block of 2**j items is a subtree (what a rank owning that
block can reduce locally). The left fold is kept only as the contrasting
schedule for tests.

``combine`` is generic over the pairwise operation, so the same schedule is
used for fp32 adds of GEMM partials, the (m, s) LSE merge of vocabulary
chunks, the (m, l, o) merge of attention splits and the MoE combine.
"""

from functools import reduce

BALANCED = "balanced"
LEFT_FOLD = "left_fold"


def balanced(items, op):
    """op-combine ``items`` by recursive halving, left half = first ceil(n/2)."""
    n = len(items)
    if n == 0:
        raise ValueError("empty tree")
    if n == 1:
        return items[0]
    h = (n + 1) // 2
    return op(balanced(items[:h], op), balanced(items[h:], op))


def left_fold(items, op):
    """(((x0 op x1) op x2) ...) op x_{n-1}."""
    if len(items) == 0:
        raise ValueError("empty tree")
    return reduce(op, items)


def combine(items, op, schedule=BALANCED):
    if schedule == BALANCED:
        return balanced(list(items), op)
    if schedule == LEFT_FOLD:
        return left_fold(list(items), op)
    raise ValueError(f"unknown schedule {schedule!r}")
