"""GPU parity of global gradient-norm clipping across shards against the oracle.

* tiny MLP, FLAT, N=4, every rank on one device: each rank's fp64 sum of
  squares, the global norm and coefficient from the four (the all-reduce's
  sum), and the clipped AdamW step, all against oracle.clip / oracle.step;
  the per-rank sums add up to the unsharded norm of the mean gradient;
* a clip coefficient of exactly 1 gives bit-identical results to the plain
  fused step; the reduction is deterministic run to run;
* the 7B rank shard at full size: the fp64 sum of squares equals the float64
  sum of the squares of the stored reduced gradient, and sampled elements of
  the clipped step match the oracle.
"""

import math

import numpy as np
import pytest
import torch

from oracle import clip as C
from oracle import step as O
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS
from tests import parity as PR

pytestmark = pytest.mark.gpu


def _replica_equal(name, st, p0, m0, v0, sl, valid, t, hp, coef, idx=None):
    """The clipped update, bit for bit against the kernel's stated fp32
    sequence: the stored fp32 mean gradient times the fp32 coefficient."""
    rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, sl, valid, t, hp, grad_scale=coef)
    for nm, got, want in (("p", st.master, rp), ("m", st.exp_avg, rm), ("v", st.exp_avg_sq, rv)):
        g = (got if idx is None else got[idx]).cpu().numpy()[:valid]
        bad = g.view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), f"{name} {nm}: {bad.sum()} elements differ from the fp32 replica"


def _clipped_round(states, max_norm, t, dev):
    """One clipped step over several ranks held on one device."""
    n = len(states)
    sq = torch.zeros(n, dtype=torch.float64, device=dev)
    for i, st in enumerate(states):
        st.plan.reduce_sqnorm(sq[i:i + 1])
    coef = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    norm = torch.zeros(1, dtype=torch.float64, device=dev)
    from rank_step_amd import binding as B
    B.fsdp_clip_coef(coef, norm, sq, n, max_norm)
    for st in states:
        st.plan.step_clipped(st.w.hparams, t, coef)
    torch.cuda.synchronize()
    return sq.cpu().numpy(), float(norm.item()), float(coef.item())


def test_tiny_mlp_clipped_every_rank(gpu):
    w = WORKLOADS[1]
    states = []
    for r in range(w.world_size):
        st = RankState(w, r, gpu, bf16_out=True, grad_out=True)
        st.make_plan()
        states.append(st)
    for t in range(1, w.steps + 1):
        snaps = []
        for st in states:
            st.load_grads(t)
            snaps.append((PR.f64(st.master), PR.f64(st.exp_avg), PR.f64(st.exp_avg_sq),
                          PR.widen_slices(st.slices, w.slice_dtype)))
        # a max_norm below the norm, so the coefficient really clips
        G = [O.reduce_mean(s[3][:, :st.segments[0][2]]) for s, st in zip(snaps, states)]
        ref_sq = [C.sq_norm(g) for g in G]
        max_norm = 0.5 * math.sqrt(math.fsum(ref_sq))
        sq, norm, coef = _clipped_round(states, max_norm, t, gpu)
        ref_norm, ref_coef = C.clip_coef(ref_sq, max_norm)
        assert ref_coef < 1.0
        for i, st in enumerate(states):
            own = PR.f64(st.grad_out)[:st.segments[0][2]]
            # the reduction of the GPU's own gradient: exact squares, fp64 sums
            assert abs(sq[i] - math.fsum((own * own).tolist())) <= 1e-12 * sq[i]
            s_g = np.mean(np.abs(snaps[i][3]), axis=0)
            assert abs(sq[i] - ref_sq[i]) <= 2e-6 * math.fsum((s_g * s_g).tolist())
        # the all-reduce stand-in: the per-rank sums add to the unsharded norm
        G_all = O.reduce_mean(np.concatenate([s[3] for s in snaps], axis=1))
        assert abs(norm - math.sqrt(C.sq_norm(G_all))) <= 2e-6 * norm
        assert abs(norm - ref_norm) <= 2e-6 * ref_norm
        own_norm, own_coef = C.clip_coef(sq.tolist(), max_norm)
        assert abs(norm - own_norm) <= 1e-13 * own_norm
        assert abs(coef - own_coef) <= 2.0 ** -23 * own_coef     # fp32 rounding of the coefficient
        for i, (st, snap) in enumerate(zip(states, snaps)):
            p0, m0, v0, sl = snap
            held = st.segments[0][2]
            ref = O.rank_step(p0, m0, v0, sl, held, t, w.hparams, grad_scale=coef)
            fl = PR.floors(p0, m0, v0, sl * coef, ref, w.hparams, t)
            gp = st.master.cpu().numpy()
            PR.assert_close(f"clip rank {i} t={t} p", gp, ref["p"], fl["p"])
            PR.assert_close(f"clip rank {i} t={t} m", st.exp_avg.cpu().numpy(), ref["m"], fl["m"])
            PR.assert_close(f"clip rank {i} t={t} v", st.exp_avg_sq.cpu().numpy(), ref["v"], fl["v"])
            PR.check_bf16(f"clip rank {i} t={t} bf16", PR.bf16_bits(st.ag_slot), gp, ref["p"], fl["p"])
            _replica_equal(f"clip rank {i} t={t}", st, p0, m0, v0, sl, held, t, w.hparams, coef)
    for st in states:
        st.close()


def test_unit_coefficient_is_the_fused_step_bitwise(gpu):
    w = WORKLOADS[3]
    a = RankState(w, 0, gpu, bf16_out=True, grad_out=True)
    b = RankState(w, 0, gpu, bf16_out=True, grad_out=True)
    a.make_plan()
    b.make_plan()
    for t in (1, 2):
        a.load_grads(t)
        b.load_grads(t)
        a.step(t)
        sq, norm, coef = _clipped_round([b], 1e30, t, gpu)
        assert coef == 1.0
        for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq),
                     (a.grad_out, b.grad_out)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(a.ag.view(torch.int16), b.ag.view(torch.int16))
    # the sum of squares is deterministic
    s1 = torch.zeros(1, dtype=torch.float64, device=gpu)
    s2 = torch.zeros(1, dtype=torch.float64, device=gpu)
    b.plan.reduce_sqnorm(s1)
    b.plan.reduce_sqnorm(s2)
    torch.cuda.synchronize()
    assert s1.view(torch.int64).item() == s2.view(torch.int64).item()
    a.close()
    b.close()


def test_llama7b_clipped_full_size(gpu):
    w = WORKLOADS[4]
    st = RankState(w, 0, gpu, bf16_out=True, grad_out=True)
    st.make_plan()
    rng = np.random.default_rng(4)
    idx = torch.from_numpy(np.unique(rng.integers(0, st.total, 1 << 20))).to(gpu)
    st.load_grads(1)
    before = (PR.f64(st.master[idx]), PR.f64(st.exp_avg[idx]), PR.f64(st.exp_avg_sq[idx]),
              PR.widen_slices(st.slices[:, idx], w.slice_dtype))
    sq, norm, coef = _clipped_round([st], 1.0, 1, gpu)
    g = st.grad_out.double()
    own = float((g * g).sum().item())       # float64 sum of the exact squares, on the device
    del g
    assert abs(sq[0] - own) <= 1e-10 * own
    own_norm, own_coef = C.clip_coef(sq.tolist(), 1.0)
    assert abs(norm - own_norm) <= 1e-13 * own_norm
    assert abs(coef - own_coef) <= 2.0 ** -23 * own_coef
    assert coef < 1.0
    p0, m0, v0, sl = before
    ref = O.rank_step(p0, m0, v0, sl, p0.size, 1, w.hparams, grad_scale=coef)
    fl = PR.floors(p0, m0, v0, sl * coef, ref, w.hparams, 1)
    gp = PR.f64(st.master[idx])
    PR.assert_close("7b clipped p", gp, ref["p"], fl["p"])
    PR.assert_close("7b clipped m", PR.f64(st.exp_avg[idx]), ref["m"], fl["m"])
    PR.assert_close("7b clipped v", PR.f64(st.exp_avg_sq[idx]), ref["v"], fl["v"])
    PR.check_bf16("7b clipped bf16", PR.bf16_bits(st.ag_slot[idx]), gp, ref["p"], fl["p"])
    _replica_equal("7b clipped", st, p0, m0, v0, sl, p0.size, 1, w.hparams, coef, idx)
    st.close()
    del st
    torch.cuda.empty_cache()
