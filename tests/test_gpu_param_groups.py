"""GPU: parameter groups as plans.

A plan steps with one set of hyperparameters, so a rank whose shards belong
to different groups (torch's param_groups; here weight decay 0.01 on the
matrices and none on the norm weights) builds one plan per group and makes
one step call per plan.  On the Llama-7B block at N = 8 (Shard(0), 8 bf16
slices):
  * eager steps, t = 1..3: every element of each group's shards against the
    oracle's step with that group's hyperparameters (per-step resync), the
    bf16 copy included; a step with the other group's weight decay would miss
    the norm weights (1.0) by 1e-5, five times the allowance;
  * the _capturable calls with one device step count per plan, both captured
    in one HIP graph and replayed with synchronisations between replays: bit
    for bit the eager fixed-count calls at every t, each count ending at the
    number of replays.
"""

import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import cstep as OC
from rank_step_amd import binding as B
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS
from tests import fullcheck as FC

pytestmark = pytest.mark.gpu

STEPS = 3


def _groups(st):
    """(decay group, no-decay group) of the rank's shards, with their
    hyperparameters: the norm weights take no weight decay."""
    hp = st.w.hparams
    no_decay = dict(hp, weight_decay=0.0)
    recs = st.mt_tensors(with_grad_out=False)
    dec = [(s, r) for s, r in zip(st.segments, recs) if not s[3]]
    nod = [(s, r) for s, r in zip(st.segments, recs) if s[3]]
    assert dec and nod, "the block has both matrices and norm weights"
    return [(dec, hp), (nod, no_decay)]


def _plans(st, groups):
    return [B.MtPlan([r for _, r in g], st.w.n_slices, st.w.slice_dtype) for g, _ in groups]


def _host(x):
    return x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.cpu().numpy()


def _check_groups(st, pre, t, groups, name, block=1 << 21):
    """Every element of each group's shards against the oracle's compiled
    step with the group's hyperparameters, block by block on the host."""
    tasks = []
    for g, hp in groups:
        for (off, length, held, _), _ in g:
            assert held == length, "the Llama block's shards have no padding"
            tasks += [(a, min(a + block, off + length), hp) for a in range(off, off + length, block)]

    def task(x):
        a, b, hp = x
        p0, m0, v0 = (_host(y[a:b]) for y in pre)
        raw = _host(st.slices[:, a:b])
        ref = OC.rank_step(p0, m0, v0, raw, "bf16", t, hp)
        return FC.check_block(a, p0, m0, v0, raw, "bf16", t, hp, ref, _host(st.master[a:b]),
                              _host(st.exp_avg[a:b]), _host(st.exp_avg_sq[a:b]),
                              gpu_bf16=_host(st.ag_slot[a:b]))

    t0 = time.perf_counter()
    stats = FC.new_stats()
    with ThreadPoolExecutor(8) as ex:
        for s in ex.map(task, tasks):
            FC.merge(stats, s)
    d = FC.assert_ok(name, stats, check_bf16=True)
    n = sum(b - a for a, b, _ in tasks)
    assert n == st.total
    print(f"{name}: every element ({n:,}) in {time.perf_counter() - t0:.1f} s; worst share of the "
          f"allowance " + " ".join(f"{k}={d[k]['worst']:.3g}" for k in ("p", "m", "v")), flush=True)


def test_groups_against_the_oracle(gpu):
    w = WORKLOADS[3]
    st = RankState(w, 0, gpu, bf16_out=True)
    groups = _groups(st)
    plans = _plans(st, groups)
    for t in range(1, STEPS + 1):
        st.load_grads(t)
        pre = (st.master.clone(), st.exp_avg.clone(), st.exp_avg_sq.clone())
        for plan, (_, hp) in zip(plans, groups):
            plan.step(hp, t)
        torch.cuda.synchronize()
        _check_groups(st, pre, t, groups, f"param groups t={t}")
        del pre
    for plan in plans:
        plan.close()


def _bits(x):
    return x.view(torch.int16) if x.element_size() == 2 else x.view(torch.int32)


def test_groups_in_one_graph_with_a_count_each(gpu):
    w = WORKLOADS[3]
    a = RankState(w, 0, gpu, bf16_out=True)
    b = RankState(w, 0, gpu, bf16_out=True)
    ga, gb = _groups(a), _groups(b)
    pa, pb = _plans(a, ga), _plans(b, gb)
    counts = [torch.zeros(1, dtype=torch.int64, device=gpu) for _ in pb]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for plan, (_, hp), count in zip(pb, gb, counts):
            plan.step_capturable(hp, count)
    torch.cuda.synchronize()
    assert all(int(c.item()) == 0 for c in counts), "capture ran the launches"
    for t in range(1, STEPS + 1):
        a.load_grads(t)
        b.load_grads(t)
        for plan, (_, hp) in zip(pa, ga):
            plan.step(hp, t)
        g.replay()
        torch.cuda.synchronize()
        for nm in ("master", "exp_avg", "exp_avg_sq", "ag_slot"):
            assert torch.equal(_bits(getattr(a, nm)), _bits(getattr(b, nm))), f"replay {t}: {nm} differs"
        assert [int(c.item()) for c in counts] == [t, t]
    del g
    for plan in pa + pb:
        plan.close()
