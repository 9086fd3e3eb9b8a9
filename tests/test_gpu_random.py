"""Seeded random plans of the fused multi-tensor step against the oracle.

Each plan draws its own shard table: the number of shards, their sizes
(empty, a few elements, several 2048-element chunk entries), how much of each
is padding, buffer offsets that keep or break the vector alignments, slice
strides wider than the shard, the slice count N and dtype, which shards write
the bf16 copy and the reduced gradient, and the AdamW hyperparameters and step.
Every shard is checked against the float64 oracle (per-step resync) with guard
words around every buffer, over two consecutive steps.
"""

import numpy as np
import pytest
import torch

from rank_step_amd import binding as B
from tests.test_gpu_kernels import Shard

pytestmark = pytest.mark.gpu

N_PLANS = 16


def _f32(x):
    return float(np.float32(x))


def _draw_plan(rng):
    n_shards = int(rng.integers(1, 25))
    specs = []
    for _ in range(n_shards):
        kind = rng.random()
        if kind < 0.06:
            S = 0
        elif kind < 0.3:
            S = int(rng.integers(1, 300))
        elif kind < 0.8:
            S = int(rng.integers(300, 6000))
        else:
            S = int(rng.integers(6000, 40000))
        valid = S if rng.random() < 0.6 else int(rng.integers(0, S + 1))
        offset = int(rng.choice([0, 0, 0, 1, 2, 4]))
        stride_extra = int(rng.choice([0, 0, 0, 1, 2, 4, 37]))
        specs.append((S, valid, offset, stride_extra, bool(rng.random() < 0.7),
                      bool(rng.random() < 0.5)))
    N = int(rng.choice([1, 2, 3, 5, 7, 8, 12]))
    sdt = str(rng.choice(["f32", "bf16"]))
    hp = dict(lr=_f32(10 ** rng.uniform(-5, -2)), beta1=_f32(rng.uniform(0.8, 0.95)),
              beta2=_f32(rng.uniform(0.95, 0.9999)), eps=_f32(10 ** rng.uniform(-10, -6)),
              weight_decay=_f32(rng.uniform(0.0, 0.1)))
    t0 = int(rng.choice([1, 2, 7, 100]))
    return specs, N, sdt, hp, t0


@pytest.mark.parametrize("plan_id", range(N_PLANS))
def test_random_plan(gpu, plan_id):
    rng = np.random.default_rng(20_000 + plan_id)
    specs, N, sdt, hp, t0 = _draw_plan(rng)
    label = f"plan {plan_id} (N={N} {sdt} {len(specs)} shards t0={t0})"
    print(label, flush=True)
    shards = [Shard(S, va, N, sdt, gpu, seed=40_000 + 100 * plan_id + i, offset=o,
                    stride_extra=x, bf16=bf, gout=go)
              for i, (S, va, o, x, bf, go) in enumerate(specs)]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    info = plan.info()
    assert info["n_tensors"] == len(specs)
    assert info["total_numel"] == sum(s[0] for s in specs)
    for t in (t0, t0 + 1):
        for i, s in enumerate(shards):
            g = torch.Generator(device=gpu)
            g.manual_seed(50_000 + 1000 * plan_id + 10 * t + i)
            x = torch.randn(N, s.S, generator=g, device=gpu) * 1e-2
            s.sl.t.view(N, s.stride)[:, :s.valid] = x[:, :s.valid].to(s.sl.t.dtype)
        snaps = [s.snapshot() for s in shards]
        plan.step(hp, t)
        torch.cuda.synchronize()
        for i, (s, snap) in enumerate(zip(shards, snaps)):
            s.check(f"{label} shard {i} t={t}", snap, t, hp=hp)
    plan.close()
