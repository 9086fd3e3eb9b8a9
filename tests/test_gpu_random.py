"""Seeded random plans of the fused multi-tensor step against the oracle.

Each plan draws its own shard table: the number of shards, their sizes
(empty, a few elements, several 2048-element chunk entries), how much of each
is padding, buffer offsets (one for the whole shard, or one per buffer, so
that shards split, read shifted slices, store copies in pieces or run
element by element), slice strides wider than the shard, the slice count N and dtype, which shards write
the bf16 copy and the reduced gradient, and the AdamW hyperparameters and step.
Every shard is checked against the float64 oracle (per-step resync) with guard
words around every buffer, over two consecutive steps.  The same random tables
drive the accumulated and clipped step and the one-pass fp8 step.  In the
fused-step plans about 30 % of the shards name their slices through tables
of pointers to separate buffers.
"""

import math

import numpy as np
import pytest
import torch

from oracle import accum as A
from oracle import fp8 as F
from oracle import step as O
from rank_step_amd import binding as B
from tests import parity as PR
from tests.test_gpu_kernels import Shard
from tests.test_gpu_slice_table import _tabled

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
        kind = rng.random()
        if kind < 0.6:      # every buffer at one offset
            offset = int(rng.choice([0, 0, 0, 1, 2, 4]))
        elif kind < 0.85:   # fp32 buffers in one phase, slices and copy anywhere
            co = int(rng.integers(0, 4))
            offset = {"p": co, "m": co, "v": co, "gout": co,
                      "sl": int(rng.integers(0, 4)), "out": int(rng.integers(0, 4))}
        else:               # every buffer anywhere (fp32 phases may disagree)
            offset = {k: int(rng.integers(0, 4)) for k in ("p", "m", "v", "gout", "sl", "out")}
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
    # about 30 % of the shards name their slices through a table of pointers
    # (separate buffers, half of them misaligned for the vector path)
    trng = np.random.default_rng(60_000 + plan_id)
    tables, recs = {}, []
    for i, s in enumerate(shards):
        if trng.random() < 0.3:
            tables[i], rec = _tabled(s, gpu, misalign=bool(trng.random() < 0.5))
            recs.append(rec)
        else:
            recs.append(s.mt())
    print(f"  {len(tables)} shards through slice tables", flush=True)
    plan = B.MtPlan(recs, N, sdt)
    del recs
    info = plan.info()
    assert info["n_tensors"] == len(specs)
    assert info["total_numel"] == sum(s[0] for s in specs)
    for t in (t0, t0 + 1):
        for i, s in enumerate(shards):
            g = torch.Generator(device=gpu)
            g.manual_seed(50_000 + 1000 * plan_id + 10 * t + i)
            x = torch.randn(N, s.S, generator=g, device=gpu) * 1e-2
            s.sl.t.view(N, s.stride)[:, :s.valid] = x[:, :s.valid].to(s.sl.t.dtype)
            for q, buf in enumerate(tables.get(i, ())):
                buf.t.copy_(s.sl.t.view(N, s.stride)[q, :s.S])
        snaps = [s.snapshot() for s in shards]
        plan.step(hp, t)
        torch.cuda.synchronize()
        for i, (s, snap) in enumerate(zip(shards, snaps)):
            s.check(f"{label} shard {i} t={t}", snap, t, hp=hp, widen=True)
        for i, bufs in tables.items():
            for buf in bufs:
                buf.check_guards(f"{label} shard {i} slice buffer")
    plan.close()


def _set_slices(shards, N, gpu, seed):
    for i, s in enumerate(shards):
        g = torch.Generator(device=gpu)
        g.manual_seed(seed + i)
        x = torch.randn(N, s.S, generator=g, device=gpu) * 1e-2
        s.sl.t.view(N, s.stride)[:, :s.valid] = x[:, :s.valid].to(s.sl.t.dtype)


N_PLANS_OTHER = 8


@pytest.mark.parametrize("plan_id", range(N_PLANS_OTHER))
def test_random_plan_accumulate_and_clip(gpu, plan_id):
    """Two micro-batches reduced and accumulated into the stored gradient (with
    the rank's sum of squares), a clip coefficient below 1, and the clipped
    update from the stored gradient: the gradient against the oracle's
    synchronised accumulation, the sum of squares against the exact squares of
    the stored values, and the update against the oracle and bit for bit
    against the kernel's stated fp32 sequence."""
    rng = np.random.default_rng(30_000 + plan_id)
    specs, N, sdt, hp, t = _draw_plan(rng)
    label = f"plan {plan_id} (N={N} {sdt} {len(specs)} shards t={t})"
    print(label, flush=True)
    shards = [Shard(S, va, N, sdt, gpu, seed=60_000 + 100 * plan_id + i, offset=o,
                    stride_extra=x, bf16=bf, gout=True)
              for i, (S, va, o, x, bf, _) in enumerate(specs)]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    micro = []
    for k in range(2):
        _set_slices(shards, N, gpu, 70_000 + 1000 * plan_id + 100 * k)
        micro.append([PR.widen_slices(s.sl.t.view(N, s.stride)[:, :s.S], sdt) for s in shards])
        sq = torch.full((1,), float("nan"), dtype=torch.float64, device=gpu)
        plan.reduce_accumulate(k, sq if k == 1 else None)
    torch.cuda.synchronize()
    sq_gpu = float(sq.item())
    own_sq = 0.0
    for i, s in enumerate(shards):
        va = s.valid
        g = s.gout.t.cpu().numpy()
        ref = A.synchronised([micro[0][i][:, :va], micro[1][i][:, :va]])
        floor = (np.abs(micro[0][i][:, :va]).sum(0) + np.abs(micro[1][i][:, :va]).sum(0)) / N
        PR.assert_close(f"{label} shard {i} accumulated g", g[:va], ref, floor)
        PR.check_pad_zero(f"{label} shard {i} g", g, va)
        own_sq = math.fsum([own_sq] + (g[:va].astype(np.float64) ** 2).tolist())
    assert abs(sq_gpu - own_sq) <= 1e-12 * own_sq, (label, sq_gpu, own_sq)
    if own_sq == 0.0:
        plan.close()
        return
    coef = torch.full((1,), float("nan"), dtype=torch.float32, device=gpu)
    max_norm = 0.3 * math.sqrt(own_sq)
    B.fsdp_clip_coef(coef, None, sq, 1, max_norm)
    snaps = []
    for s in shards:
        g = PR.f64(s.gout.t)
        snaps.append((PR.f64(s.p.t), PR.f64(s.m.t), PR.f64(s.v.t), g[None, :]))
    plan.step_clipped(hp, t, coef)
    torch.cuda.synchronize()
    c = float(coef.item())
    assert c < 1.0 and abs(c - max_norm / (math.sqrt(own_sq) + 1e-6)) <= 2.0 ** -23 * c
    for i, (s, (p0, m0, v0, g1)) in enumerate(zip(shards, snaps)):
        va = s.valid
        ref = O.rank_step(p0, m0, v0, g1, va, t, hp, grad_scale=c)
        fl = PR.floors(p0[:va], m0[:va], v0[:va], g1[:, :va] * c,
                       {k: r[:va] for k, r in ref.items()}, hp, t, widen=True)
        gp = s.p.t.cpu().numpy()
        PR.assert_close(f"{label} shard {i} p", gp[:va], ref["p"][:va], fl["p"])
        PR.assert_close(f"{label} shard {i} m", s.m.t.cpu().numpy()[:va], ref["m"][:va], fl["m"])
        PR.assert_close(f"{label} shard {i} v", s.v.t.cpu().numpy()[:va], ref["v"][:va], fl["v"])
        rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, g1, va, t, hp, grad_scale=c)
        for nm, got, want in (("p", s.p.t, rp), ("m", s.m.t, rm), ("v", s.v.t, rv)):
            bad = got.cpu().numpy()[:va].view(np.uint32) != want.view(np.uint32)
            assert not bad.any(), f"{label} shard {i} {nm}: {bad.sum()} differ from the fp32 replica"
        for b, nm in ((s.p, "p"), (s.m, "m"), (s.v, "v")):
            PR.check_pad_zero(f"{label} shard {i} {nm}", b.t.cpu().numpy(), va)
        if s.out is not None:
            bits = PR.bf16_bits(s.out.t)
            PR.check_bf16(f"{label} shard {i} bf16", bits[:va], gp[:va], ref["p"][:va], fl["p"])
            PR.check_pad_zero(f"{label} shard {i} bf16", bits, va)
        for b in s.bufs():
            b.check_guards(label)
    plan.close()


@pytest.mark.parametrize("plan_id", range(N_PLANS_OTHER))
def test_random_plan_fp8_delayed_scaling(gpu, plan_id):
    """The one-pass fp8 step with scales fixed before it: fp32 state, bf16
    copies and stored gradients bit-identical to the plain fused step on the
    same inputs; each shard's amax the largest |p'| of the GPU's own update
    (fp32 bits); every code the oracle's quantisation of that p' with the
    given scale; zero codes in the padding and no byte written outside."""
    rng = np.random.default_rng(40_000 + plan_id)
    specs, N, sdt, hp, t = _draw_plan(rng)
    label = f"plan {plan_id} (N={N} {sdt} {len(specs)} shards t={t})"
    print(label, flush=True)

    def make():
        return [Shard(S, va, N, sdt, gpu, seed=80_000 + 100 * plan_id + i, offset=o,
                      stride_extra=x, bf16=bf, gout=go)
                for i, (S, va, o, x, bf, go) in enumerate(specs)]
    a, b = make(), make()
    f8 = []
    for s in a:
        off = int(rng.integers(0, 4))
        full = torch.full((s.S + off + 16,), 0xAB, dtype=torch.uint8, device=gpu)
        f8.append((full, off, full[off:off + s.S]))
    ta = [dict(s.mt(), unshard_fp8_out=f[2]) for s, f in zip(a, f8)]
    plan_a = B.MtPlan(ta, N, sdt)
    plan_b = B.MtPlan([s.mt() for s in b], N, sdt)
    n = len(specs)
    scales = np.float32(448.0) / rng.uniform(0.005, 0.2, n).astype(np.float32)
    scales[rng.random(n) < 0.15] = np.float32(1e30)      # most values saturate
    scale_in = torch.from_numpy(scales).to(gpu)
    amax = torch.full((n,), -1.0, dtype=torch.float32, device=gpu)
    _set_slices(a, N, gpu, 90_000 + 1000 * plan_id)
    _set_slices(b, N, gpu, 90_000 + 1000 * plan_id)
    plan_a.step_fp8(hp, t, scale_in, amax)
    plan_b.step(hp, t)
    torch.cuda.synchronize()
    am = amax.cpu().numpy()
    for i, (x, y) in enumerate(zip(a, b)):
        for nm in ("p", "m", "v", "gout"):
            bx, by = getattr(x, nm), getattr(y, nm)
            if bx is not None:
                assert torch.equal(bx.t.view(torch.int32), by.t.view(torch.int32)), (label, i, nm)
        if x.out is not None:
            assert torch.equal(x.out.t.view(torch.int16), y.out.t.view(torch.int16)), (label, i)
        va = x.valid
        p = x.p.t.cpu().numpy()
        want = np.float32(np.abs(p[:va]).max()) if va else np.float32(0.0)
        assert am[i].view(np.uint32) == want.view(np.uint32), (label, i, am[i], want)
        full, off, codes_t = f8[i]
        codes = codes_t.cpu().numpy().astype(np.uint8)
        ref = F.quantize(p[:va], scales[i])
        assert np.array_equal(codes[:va], ref), (label, i)
        assert np.all(codes[va:] == 0), (label, i)
        rest = full.cpu().numpy()
        assert np.all(rest[:off] == 0xAB) and np.all(rest[off + x.S:] == 0xAB), (label, i)
    plan_a.close()
    plan_b.close()
