"""GPU parity on the five synthetic workloads, in the launch configuration the
benchmark times (one multi-tensor plan over the rank's packed shards).

* tiny MLP, FLAT, N=4: every rank, every element, 3 steps, per-step resync and
  a free-running double-precision trajectory beside it; the other ranks' slots
  of the packed all-gather buffer stay untouched.
* 128 MiB MLP, FLAT, N=4 (rank 0): every element, 10 steps, resync and
  free-running.
* Llama-7B block, Shard(0), N=8: every element of all 5 steps (resync), and
  the oracle's own trajectory over every element beside it (free-running).
* 7B rank shard (291 shards, 842,301,952 params, 5 steps) and 70B rank shard
  (723 shards, 2,204,803,328 params, 3 steps): every element of every step
  (resync); at every step also a sample of elements (random plus the first
  and last of every shard) bit for bit against the kernel's fp32 sequence,
  and the oracle's own trajectory from the initial state on that sample
  (free-running).
* Units of odd sizes (FLAT N=4, Shard(0) N=8), every rank and element: shard
  sizes that are not multiples of 4, so slices sit at odd strides, all-gather
  slots and packed shards start off vector boundaries.

The full-size checks run the oracle's compiled step (oracle/rank_step.c, bit
for bit oracle.step) and the C form of the parity rules (tests/c/fullcheck.c)
over blocks of the rank's buffer on the host's threads, and print, per
checked step, the elapsed time, the largest share of the mixed allowance each
output uses, the elements outside the literal 2e-6 relative bound, and the
bf16 words that differ from RNE of the oracle's value.
"""

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import cstep as OC
from oracle import layout as OL
from oracle import step as O
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS, Param, Workload, shapes_of
from tests import fullcheck as FC
from tests import parity as PR

pytestmark = pytest.mark.gpu


def _layout_matches_oracle(st):
    w = st.w
    mode = {"flat": OL.FLAT, "shard0": OL.SHARD0, "owner": OL.OWNER}[w.mode]
    ref_v, ref_s = OL.layout(mode, w.world_size, st.rank, shapes_of(w), w.has_master)
    assert st.views == [v.__dict__ for v in ref_v]
    assert st.summary == ref_s.__dict__


def _report(name, worst, literal=None, bf16_diff=None, elapsed=None, n=None):
    """One line per checked step: the largest share of the mixed allowance
    each output uses (1.0 would fail), and for the full-size checks the
    elements outside the literal relative bound and the bf16 words that
    differ from RNE(oracle)."""
    parts = [f"{name}:"]
    if n is not None:
        parts.append(f"every element ({n:,})" + (f" in {elapsed:.1f} s;" if elapsed is not None else ";"))
    parts.append("worst share of the allowance " + " ".join(f"{k}={v:.3g}" for k, v in worst.items()) + ";")
    if literal is not None:
        parts.append("beyond the literal 2e-6 bound " + " ".join(f"{k}={v}" for k, v in literal.items()) + ";")
    if bf16_diff is not None:
        parts.append(f"bf16 != RNE(oracle): {bf16_diff}")
    print(" ".join(parts), flush=True)


def _check_full(st, snap, t, name, check_g=False):
    p0, m0, v0, sl = snap
    hp = st.w.hparams
    gp = st.master.cpu().numpy()
    gm = st.exp_avg.cpu().numpy()
    gv = st.exp_avg_sq.cpu().numpy()
    bits = PR.bf16_bits(st.ag_slot) if st.ag_slot is not None else None
    worst = {"p": 0.0, "m": 0.0, "v": 0.0}
    if check_g:
        worst["g"] = 0.0
    for off, length, held, _ in st.segments:
        a, b = off, off + held
        ref = O.rank_step(p0[a:b], m0[a:b], v0[a:b], sl[:, a:b], held, t, hp)
        fl = PR.floors(p0[a:b], m0[a:b], v0[a:b], sl[:, a:b], ref, hp, t)
        for nm, arr in (("p", gp), ("m", gm), ("v", gv)):
            PR.assert_close(f"{name} {nm}", arr[a:b], ref[nm], fl[nm])
            worst[nm] = max(worst[nm], PR.mixed_ratio(arr[a:b], ref[nm], fl[nm]))
            PR.check_pad_zero(f"{name} {nm}", arr[a:off + length], held)
        if bits is not None:
            PR.check_bf16(f"{name} bf16", bits[a:b], gp[a:b], ref["p"], fl["p"])
            PR.check_pad_zero(f"{name} bf16", bits[a:off + length], held)
        if check_g:
            gg = st.grad_out.cpu().numpy()
            PR.assert_close(f"{name} g", gg[a:b], ref["g"], fl["g"])
            worst["g"] = max(worst["g"], PR.mixed_ratio(gg[a:b], ref["g"], fl["g"]))
    _report(name, worst)
    return worst


def _snapshot(st):
    return (PR.f64(st.master), PR.f64(st.exp_avg), PR.f64(st.exp_avg_sq),
            PR.widen_slices(st.slices, st.w.slice_dtype))


def test_tiny_mlp_every_rank(gpu):
    w = WORKLOADS[1]
    for r in range(w.world_size):
        st = RankState(w, r, gpu, bf16_out=True, grad_out=True, ag_full=True)
        _layout_matches_oracle(st)
        assert st.total == 147_520 and len(st.segments) == 1
        st.make_plan()
        free = None
        for t in range(1, w.steps + 1):
            st.load_grads(t)
            snap = _snapshot(st)
            if free is None:
                free = snap[:3]
                ffl = {"p": np.abs(free[0]), "m": np.abs(free[1]), "v": free[2]}
            st.step(t)
            torch.cuda.synchronize()
            _check_full(st, snap, t, f"tiny rank {r} t={t}", check_g=True)
            # free-running double trajectory from the initial state
            ref = O.rank_step(*free, snap[3], st.total, t, w.hparams)
            free = (ref["p"], ref["m"], ref["v"])
            ffl = fl = PR.free_floors(ffl, snap[3], ref, w.hparams, t)
            PR.assert_close(f"tiny rank {r} free p t={t}", st.master.cpu().numpy(), ref["p"], fl["p"])
            PR.assert_close(f"tiny rank {r} free m t={t}", st.exp_avg.cpu().numpy(), ref["m"], fl["m"])
            PR.assert_close(f"tiny rank {r} free v t={t}", st.exp_avg_sq.cpu().numpy(), ref["v"], fl["v"])
        # the other ranks' slots of the packed all-gather buffer are untouched (zeros)
        ag = PR.bf16_bits(st.ag)
        S = st.total
        mask = np.ones(ag.size, dtype=bool)
        mask[r * S:(r + 1) * S] = False
        assert np.all(ag[mask] == 0)
        st.close()


def test_mlp128m_rank0(gpu):
    w = WORKLOADS[2]
    st = RankState(w, 0, gpu, bf16_out=True)
    _layout_matches_oracle(st)
    assert st.total == 8_388_608
    st.make_plan()
    free = None
    for t in range(1, w.steps + 1):
        st.load_grads(t)
        snap = _snapshot(st)
        assert (snap[3] == 0).mean() > 0.09          # 10% exact zeros per slice
        if free is None:
            free = snap[:3]
            ffl = {"p": np.abs(free[0]), "m": np.abs(free[1]), "v": free[2]}
        st.step(t)
        torch.cuda.synchronize()
        _check_full(st, snap, t, f"mlp128m t={t}")
        ref = O.rank_step(*free, snap[3], st.total, t, w.hparams)
        free = (ref["p"], ref["m"], ref["v"])
        ffl = PR.free_floors(ffl, snap[3], ref, w.hparams, t)
        _free_check(st, None, ref, ffl, f"mlp128m free t={t}")
        del snap, ref
    st.close()


def _free_check(st, idx_t, ref, ffl, name):
    """The GPU's state (all of it, or the elements idx_t) against the
    oracle's own trajectory, with the floors carried along it."""
    worst = {}
    for nm, t_ in (("p", st.master), ("m", st.exp_avg), ("v", st.exp_avg_sq)):
        got = (t_ if idx_t is None else t_[idx_t]).cpu().numpy()
        PR.assert_close(f"{name} {nm}", got, ref[nm], ffl[nm])
        worst[nm] = PR.mixed_ratio(got, ref[nm], ffl[nm])
    _report(name, worst)


def _host_threads():
    """Worker threads for the host-side checks: at most 16, the CPU share a
    host grants one GPU's process, whatever the affinity mask shows."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _every_element(st, pre, t, name, block=1 << 22):
    """Every element of the rank's buffer after step t against the oracle,
    from the GPU's state before the step (``pre``: device copies of master,
    exp_avg and exp_avg_sq; the slices are still in place).  The buffer has no
    padding (all five workloads divide evenly), so it is checked as one range,
    block by block on the host's threads: the oracle's compiled step and the C
    form of the parity rules, both of which release the GIL."""
    w = st.w
    hp = w.hparams
    sdt = w.slice_dtype
    assert st.summary["pad_numel"] == 0
    total = st.total
    bounds = [(a, min(a + block, total)) for a in range(0, total, block)]

    def host(x):
        return x.view(torch.int16).cpu().numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.cpu().numpy()

    def task(ab):
        a, b = ab
        p0, m0, v0 = (host(x[a:b]) for x in pre)
        raw = host(st.slices[:, a:b])
        gp, gm, gv = host(st.master[a:b]), host(st.exp_avg[a:b]), host(st.exp_avg_sq[a:b])
        bits = host(st.ag_slot[a:b]) if st.ag_slot is not None else None
        ref = OC.rank_step(p0, m0, v0, raw, sdt, t, hp)
        return FC.check_block(a, p0, m0, v0, raw, sdt, t, hp, ref, gp, gm, gv, gpu_bf16=bits)

    t0 = time.perf_counter()
    stats = FC.new_stats()
    with ThreadPoolExecutor(_host_threads()) as ex:
        for s in ex.map(task, bounds):
            FC.merge(stats, s)
    elapsed = time.perf_counter() - t0
    d = FC.assert_ok(name, stats, check_bf16=st.ag_slot is not None)
    _report(name, {k: d[k]["worst"] for k in ("p", "m", "v")},
            {k: d[k]["literal"] for k in ("p", "m", "v")},
            d["bf16"]["diff_vs_oracle"] if st.ag_slot is not None else None, elapsed, total)
    return d


def _sample_idx(st, n, seed):
    rng = np.random.default_rng(seed)
    idx = [rng.integers(0, st.total, n)]
    for off, length, held, _ in st.segments:
        idx.append(np.arange(off, off + min(16, length)))
        idx.append(np.arange(off + max(0, length - 16), off + length))
    return np.unique(np.concatenate(idx))


def _check_sampled(st, idx_t, before, t, name):
    """Oracle on the sampled elements, from the GPU's state before the step.
    (These workloads have no padding: every sampled element is valid.)"""
    p0, m0, v0, sl = before
    hp = st.w.hparams
    assert st.summary["pad_numel"] == 0
    ref = O.rank_step(p0, m0, v0, sl, p0.size, t, hp)
    fl = PR.floors(p0, m0, v0, sl, ref, hp, t)
    gp = PR.f64(st.master[idx_t])
    PR.assert_close(f"{name} p", gp, ref["p"], fl["p"])
    PR.assert_close(f"{name} m", PR.f64(st.exp_avg[idx_t]), ref["m"], fl["m"])
    PR.assert_close(f"{name} v", PR.f64(st.exp_avg_sq[idx_t]), ref["v"], fl["v"])
    if st.ag_slot is not None:
        PR.check_bf16(f"{name} bf16", PR.bf16_bits(st.ag_slot[idx_t]), gp, ref["p"], fl["p"])
    # and bit for bit against the kernel's stated fp32 sequence
    rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, sl, p0.size, t, hp)
    for nm, got, want in (("p", st.master, rp), ("m", st.exp_avg, rm), ("v", st.exp_avg_sq, rv)):
        g = got[idx_t].cpu().numpy()
        bad = g.view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), f"{name} {nm}: {bad.sum()} elements differ from the fp32 replica"


def _run_full_size(cfg, gpu, n_sample, full_steps):
    """Every step: the sampled resync check, the replica and the oracle's own
    trajectory on the sample; at ``full_steps``, every element (resync)."""
    w = WORKLOADS[cfg]
    st = RankState(w, 0, gpu, bf16_out=True)
    _layout_matches_oracle(st)
    st.make_plan()
    info = st.plan.info()
    assert info["n_tensors"] == len(st.segments)
    idx = _sample_idx(st, n_sample, cfg)
    idx_t = torch.from_numpy(idx).to(gpu)
    free = ffl = None
    for t in range(1, w.steps + 1):
        st.load_grads(t)
        pre = (st.master.clone(), st.exp_avg.clone(), st.exp_avg_sq.clone()) if t in full_steps else None
        before = (PR.f64(st.master[idx_t]), PR.f64(st.exp_avg[idx_t]), PR.f64(st.exp_avg_sq[idx_t]),
                  PR.widen_slices(st.slices[:, idx_t], w.slice_dtype))
        if free is None:
            free = before[:3]
            ffl = {"p": np.abs(free[0]), "m": np.abs(free[1]), "v": free[2]}
        st.step(t)
        torch.cuda.synchronize()
        _check_sampled(st, idx_t, before, t, f"cfg{cfg} t={t} sampled")
        ref = O.rank_step(*free, before[3], idx.size, t, w.hparams)
        free = (ref["p"], ref["m"], ref["v"])
        ffl = PR.free_floors(ffl, before[3], ref, w.hparams, t)
        _free_check(st, idx_t, ref, ffl, f"cfg{cfg} free t={t} (sample of {idx.size:,})")
        if pre is not None:
            _every_element(st, pre, t, f"cfg{cfg} t={t}")
            del pre
    st.close()
    return st


def test_llama7b_block(gpu):
    """Every element of every step, resync and free-running (the oracle's own
    trajectory over all 25,297,920 elements, in blocks on the host's threads)."""
    w = WORKLOADS[3]
    st = RankState(w, 0, gpu, bf16_out=True)
    _layout_matches_oracle(st)
    assert st.total == 25_297_920
    st.make_plan()
    block = 1 << 21
    bounds = [(a, min(a + block, st.total)) for a in range(0, st.total, block)]
    free = None
    for t in range(1, w.steps + 1):
        st.load_grads(t)
        pre = (st.master.clone(), st.exp_avg.clone(), st.exp_avg_sq.clone())
        if free is None:
            free = [(PR.f64(pre[0][a:b]), PR.f64(pre[1][a:b]), PR.f64(pre[2][a:b])) for a, b in bounds]
            ffl = [{"p": np.abs(f[0]), "m": np.abs(f[1]), "v": f[2]} for f in free]
        st.step(t)
        torch.cuda.synchronize()
        _every_element(st, pre, t, f"cfg3 t={t}")
        del pre

        def traj(i):
            a, b = bounds[i]
            raw = st.slices[:, a:b].view(torch.int16).cpu().numpy().view(np.uint16)
            ref = OC.rank_step(*free[i], raw, "bf16", t, w.hparams)
            fl = PR.free_floors(ffl[i], O.widen_bf16_bits(raw), ref, w.hparams, t)
            worst = {}
            for nm, t_ in (("p", st.master), ("m", st.exp_avg), ("v", st.exp_avg_sq)):
                got = t_[a:b].cpu().numpy()
                PR.assert_close(f"cfg3 free t={t} [{a}:{b}) {nm}", got, ref[nm], fl[nm])
                worst[nm] = PR.mixed_ratio(got, ref[nm], fl[nm])
            free[i] = (ref["p"], ref["m"], ref["v"])
            ffl[i] = fl
            return worst

        with ThreadPoolExecutor(_host_threads()) as ex:
            ws = list(ex.map(traj, range(len(bounds))))
        _report(f"cfg3 free t={t} (every element)", {k: max(x[k] for x in ws) for k in ("p", "m", "v")})
    st.close()


def test_llama7b_full_rank_shard(gpu):
    st = _run_full_size(4, gpu, 1 << 20, full_steps=range(1, 6))
    assert st.total == 842_301_952 and len(st.segments) == 291
    del st
    torch.cuda.empty_cache()


def test_llama70b_rank_shard(gpu):
    st = _run_full_size(5, gpu, 1 << 20, full_steps=range(1, 4))
    assert st.total == 2_204_803_328 and len(st.segments) == 723
    del st
    torch.cuda.empty_cache()


# odd sizes: FLAT with P = 590,081 (S = 147,521, 3 padding elements), and
# Shard(0) with rows and dim-0 sizes that leave every packed shard, its
# slices and its all-gather slot at varying element phases
ODD = {
    "flat": Workload(91, "odd_flat_n4", "flat", 4,
                     (Param("W1", (256, 256), "f32"), Param("b1", (257,), "f32"),
                      Param("W2", (1024, 256), "f32"), Param("W3", (256, 1024), "f32")),
                     "f32", 4, False, True, 2, 1e-2),
    "shard0": Workload(92, "odd_shard0_n8", "shard0", 8,
                       (Param("emb", (1001, 3), "bf16"), Param("w1", (257, 129), "bf16"),
                        Param("n1", (129,), "bf16", True), Param("w2", (77, 61), "bf16"),
                        Param("b2", (61,), "bf16"), Param("w3", (4099, 17), "bf16")),
                     "bf16", 8, True, True, 2, 1e-3),
}


@pytest.mark.parametrize("kind", ["flat", "shard0"])
def test_odd_sizes_every_rank(gpu, kind):
    w = ODD[kind]
    for r in range(w.world_size):
        st = RankState(w, r, gpu, bf16_out=True, grad_out=True, ag_full=True, garbage_pad=True)
        _layout_matches_oracle(st)
        plan = st.make_plan()
        if kind == "shard0":
            # packed shards that start off a vector boundary are split
            phases = [off % 4 for off, length, held, _ in st.segments]
            assert any(phases), "the sizes should put some shards off a vector boundary"
            entries = sum(-(-length // 2048) for _, length, _, _ in st.segments)
            assert plan.info()["n_chunks"] > entries
        for t in range(1, w.steps + 1):
            st.load_grads(t)
            snap = _snapshot(st)
            st.step(t)
            torch.cuda.synchronize()
            _check_full(st, snap, t, f"{w.name} rank {r} t={t}", check_g=True)
        ag = PR.bf16_bits(st.ag)
        S = st.total
        mask = np.ones(ag.size, dtype=bool)
        mask[r * S:(r + 1) * S] = False
        assert np.all(ag[mask] == 0), f"{w.name} rank {r}: another rank's slot written"
        st.close()
