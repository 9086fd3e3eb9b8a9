"""Oracle: gradient accumulation over micro-batches, in float64.

Test infrastructure only (see ``oracle/__init__``).

FSDP chapter §18.26 "FSDP x gradient accumulation" and §18.39: by default
every micro-batch's backward ends in a reduce-scatter and the reduced 1/N
gradient accumulates in the shard ("synchronised"); with no_sync /
set_requires_gradient_sync(False) the N-1 first micro-batches skip the
collective and each rank accumulates its unsharded gradient in place, and
only the last micro-batch reduce-scatters the accumulated sums.  Both give
the shard the same gradient, (1/N) sum_q sum_k x_{q,k}; they differ in
communication count and in memory (the unsharded gradient is N times the
shard).  Accumulation is a plain sum over micro-batches (torch adds into
.grad); scaling the loss per micro-batch is the caller's business.
"""

import numpy as np

from .step import reduce_mean


def accumulate(acc, micro):
    """In-place accumulation of one micro-batch: acc + micro (acc None = first)."""
    micro = np.asarray(micro, dtype=np.float64)
    return micro.copy() if acc is None else np.asarray(acc, dtype=np.float64) + micro


def synchronised(slices_per_micro):
    """Shard gradient when every micro-batch reduce-scatters: the sum over
    micro-batches of each micro-batch's mean over ranks.  Input: a list over
    micro-batches of [N, n] slices."""
    acc = None
    for sl in slices_per_micro:
        acc = accumulate(acc, reduce_mean(sl))
    return acc


def no_sync(slices_per_micro):
    """Shard gradient when the ranks accumulate unsharded and reduce once: the
    mean over ranks of each rank's sum over micro-batches."""
    acc = None
    for sl in slices_per_micro:
        acc = accumulate(acc, sl)
    return reduce_mean(acc)
