"""GPU parity of gradient accumulation over micro-batches.

* fsdp_grad_accumulate (no_sync, unsharded): fp32 and bf16 micro-batches,
  ragged and misaligned sizes; the first micro-batch is an exact copy, later
  ones one fp32 add each; bit-exact on values whose sums are exact;
* every rank of the tiny MLP, K=3 micro-batches per step, two steps: the
  synchronised path (reduce-accumulate into the shard, then the update from
  the stored gradient) and the no_sync path (per-rank unsharded accumulation,
  then the fused step on the accumulated slices), each against the oracle.
"""

import numpy as np
import pytest
import torch

from oracle import accum as A
from oracle import step as O
from rank_step_amd import binding as B
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS
from tests import parity as PR

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dt", ["f32", "bf16"])
# off: element offset of the accumulator; xoff: of the micro-batch gradient
# (the accumulator aligned and the gradient 1-3 elements past a vector
# boundary takes the shifted loads)
@pytest.mark.parametrize("n,off,xoff", [(0, 0, 0), (1, 0, 0), (7, 0, 0), (8, 0, 0), (2048 * 3 + 517, 0, 0),
                                        (70001, 1, 1), (4096 + 257, 2, 2), (4096 + 257, 4, 4),
                                        (4096 + 257, 0, 1), (4096 + 257, 0, 2), (70001, 0, 3)])
def test_grad_accumulate(gpu, dt, n, off, xoff):
    g = torch.Generator(device=gpu)
    g.manual_seed(n + off + 10 * xoff)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    acc_full = torch.full((n + off + 8,), float("nan"), dtype=torch.float32, device=gpu)
    acc = acc_full[off:off + n]
    ref = None
    floor = np.zeros(n)
    for k in range(4):
        x = (torch.randn(n, generator=g, device=gpu) * 10.0 ** (k - 2)).to(tdt)
        if n:
            x[0] = -0.0 if k == 0 else x[0]
        xs = torch.zeros(n + xoff, dtype=tdt, device=gpu)[xoff:]
        xs.copy_(x)
        B.fsdp_grad_accumulate(acc, xs, dt, n, k > 0)
        torch.cuda.synchronize()
        xh = PR.widen_slices(xs.view(1, n), dt)[0]
        ref = A.accumulate(ref, xh)
        floor = floor + np.abs(xh)
        got = acc.cpu().numpy()
        if k == 0:
            assert np.array_equal(got.view(np.uint32), xh.astype(np.float32).view(np.uint32))
        else:
            PR.assert_close(f"acc {dt} n={n} k={k}", got, ref, floor)
    assert torch.isnan(acc_full[off + n:]).all() and (off == 0 or torch.isnan(acc_full[:off]).all())


def test_grad_accumulate_exact_values(gpu):
    rng = np.random.default_rng(2)
    n = 5000
    m = np.round(np.ldexp(rng.uniform(0.5, 1, (6, n)), 8))
    xs = np.ldexp(m, rng.integers(-4, 4, (6, n)) - 8) * np.where(rng.random((6, n)) < 0.5, -1, 1)
    acc = torch.empty(n, dtype=torch.float32, device=gpu)
    ref = None
    for k in range(6):
        x = torch.from_numpy(xs[k].astype(np.float32)).to(gpu)
        B.fsdp_grad_accumulate(acc, x, "f32", n, k > 0)
        ref = A.accumulate(ref, xs[k])
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.float64), ref)


def _micro(w, st, t, k, dev):
    """Micro-batch k of step t: a fresh set of seeded slices for this rank."""
    from rank_step_amd.workloads import grad_slices
    return grad_slices(w, st.total, 1000 + 10 * t + k, st.rank, dev)


def test_tiny_mlp_synchronised_and_no_sync(gpu):
    w = WORKLOADS[1]
    N, K = w.world_size, 3
    one = torch.ones(1, dtype=torch.float32, device=gpu)
    for r in range(N):
        sync = RankState(w, r, gpu, bf16_out=True, grad_out=True)
        nos = RankState(w, r, gpu, bf16_out=True)
        sync.make_plan()
        nos.make_plan()
        S = sync.total
        acc = torch.empty(N, S, dtype=torch.float32, device=gpu)
        sq = torch.zeros(1, dtype=torch.float64, device=gpu)
        for t in (1, 2):
            before_s = (PR.f64(sync.master), PR.f64(sync.exp_avg), PR.f64(sync.exp_avg_sq))
            before_n = (PR.f64(nos.master), PR.f64(nos.exp_avg), PR.f64(nos.exp_avg_sq))
            micros = []
            for k in range(K):
                mk = _micro(w, sync, t, k, gpu)
                micros.append(PR.widen_slices(mk, w.slice_dtype))
                sync.slices.copy_(mk)
                sync.plan.reduce_accumulate(k > 0, sq if k == K - 1 else None)
                for q in range(N):                      # each rank's unsharded accumulation
                    B.fsdp_grad_accumulate(acc[q], mk[q], w.slice_dtype, S, k > 0)
            sync.plan.step_clipped(w.hparams, t, one)
            nos.slices.copy_(acc)                       # the one reduce-scatter's input
            nos.step(t)
            torch.cuda.synchronize()
            G_sync = A.synchronised(micros)
            G_nos = A.no_sync(micros)
            floor_g = np.sum([np.mean(np.abs(m), axis=0) for m in micros], axis=0)
            gs = sync.grad_out.cpu().numpy()
            PR.assert_close(f"sync g rank {r} t={t}", gs, G_sync, floor_g)
            assert abs(sq.item() - float(np.sum(gs.astype(np.float64) ** 2))) <= 1e-12 * sq.item()
            for name, st, G, bf in (("sync", sync, G_sync, before_s), ("no_sync", nos, G_nos, before_n)):
                p0, m0, v0 = bf
                pn, mn, vn = O.adamw(p0, m0, v0, G, t, **{k2: w.hparams[k2] for k2 in
                                                           ("lr", "beta1", "beta2", "eps", "weight_decay")})
                ref = {"p": pn, "m": mn, "v": vn}
                # floors from the micro-batch magnitudes (the accumulated gradient's terms)
                fl = PR.floors(p0, m0, v0, np.stack([floor_g]), ref, w.hparams, t)
                gp = st.master.cpu().numpy()
                PR.assert_close(f"{name} p rank {r} t={t}", gp, pn, fl["p"])
                PR.assert_close(f"{name} m rank {r} t={t}", st.exp_avg.cpu().numpy(), mn, fl["m"])
                PR.assert_close(f"{name} v rank {r} t={t}", st.exp_avg_sq.cpu().numpy(), vn, fl["v"])
                PR.check_bf16(f"{name} bf16 rank {r} t={t}", PR.bf16_bits(st.ag_slot), gp, pn, fl["p"])
        sync.close()
        nos.close()
