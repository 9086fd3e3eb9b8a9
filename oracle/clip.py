"""Oracle: global gradient-norm clipping across shards, in float64.

Test infrastructure only (see ``oracle/__init__``).

FSDP chapter §18.18 "FSDP x clip_grad_norm": with sharded gradients the
local norm is not the global norm.  Each rank takes the sum of squares of its
own gradient shard, an all-reduce sums those over the ranks, the square root
gives the global norm, and every rank scales its own shard with it -- one
scalar all-reduce, mathematically the same as clipping on one rank.  The page
names clip_grad_norm_(max_norm, norm_type=2.0) without printing its formula;
the reading taken is torch.nn.utils.clip_grad_norm_'s:

    norm  = sqrt(sum over all elements of g^2)
    coef  = min(1, max_norm / (norm + 1e-6))
    g    <- g * coef

The squared sums use math.fsum (correctly rounded), so a shard-wise sum then a
sum over ranks equals the sum over the unsharded vector exactly.
"""

import math

import numpy as np

CLIP_EPS = 1e-6


def sq_norm(g):
    """Correctly rounded sum of squares of a float64 vector (the squares of
    fp32 values are exact in float64; for float64 inputs they are rounded)."""
    g = np.asarray(g, dtype=np.float64).ravel()
    return math.fsum((g * g).tolist()) if g.size else 0.0


def clip_coef(sq_norms, max_norm):
    """Global norm from the ranks' squared norms (the all-reduce stand-in is
    the sum), and the clip coefficient; returns (norm, coef)."""
    total = math.fsum(float(x) for x in sq_norms)
    norm = math.sqrt(total)
    coef = max_norm / (norm + CLIP_EPS)
    if not math.isnan(coef):
        coef = min(1.0, coef)
    return norm, coef
