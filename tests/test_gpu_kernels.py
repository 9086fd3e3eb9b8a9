"""GPU parity of each entry point against the oracle, on small ragged shards.

Every call goes through the C ABI (rank_step_amd.binding).  Sizes span
several 2048-element chunk entries (eight 256-element workgroup tiles each)
and a ragged tail; the cases cover empty
shards, all-padding shards (valid = 0), partial groups, misaligned buffers
(element-by-element path, or a split into a short head and an aligned body
when every buffer is misaligned alike), slice strides wider than the shard,
N that is not a power of two, NaN/Inf inputs, guard words around every buffer, and the
bit-identity of the fused multi-tensor step with the chain of three calls.
"""

import numpy as np
import pytest
import torch

from oracle import step as O
from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS
from tests import parity as PR

pytestmark = pytest.mark.gpu

HP = dict(HPARAMS)
GUARD = 64
CANARY_F32 = -7.0e33


class Buf:
    """A device buffer with guard words on both sides; ``t`` is the payload view.

    ``offset`` shifts the payload by whole elements: 1 breaks every vector
    alignment, 4 keeps fp32 buffers 16-byte aligned and bf16 buffers 8-byte
    (but not 16-byte) aligned.
    """

    def __init__(self, n, dtype, device, fill=float("nan"), offset=0):
        self.n = n
        self.offset = offset
        self.full = torch.empty(n + 2 * GUARD + offset, dtype=dtype, device=device)
        self.full.fill_(CANARY_F32 if dtype == torch.float32 else 1.5)
        self.t = self.full[GUARD + offset:GUARD + offset + n]
        self.t.fill_(fill)
        self._canary = None

    def seal(self):
        self._canary = torch.cat([self.full[:GUARD + self.offset], self.full[GUARD + self.offset + self.n:]]).clone()

    def check_guards(self, name):
        now = torch.cat([self.full[:GUARD + self.offset], self.full[GUARD + self.offset + self.n:]])
        assert torch.equal(now.view(torch.int16 if now.dtype == torch.bfloat16 else torch.int32),
                           self._canary.view(torch.int16 if now.dtype == torch.bfloat16 else torch.int32)), \
            f"{name}: guard words overwritten"


class Shard:
    """One shard's buffers.  ``offset``: element offset of every buffer, or a
    dict of per-buffer offsets (keys p, m, v, sl, out, gout; default 0)."""

    def __init__(self, S, valid, N, sdt, device, seed, offset=0, stride_extra=0, bf16=True,
                 gout=True):
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        f32 = torch.float32
        off = (lambda k: offset.get(k, 0)) if isinstance(offset, dict) else (lambda k: offset)
        self.S, self.valid, self.N, self.sdt = S, valid, N, sdt
        self.p = Buf(S, f32, device, fill=1.0e30, offset=off("p"))
        self.m = Buf(S, f32, device, fill=float("nan"), offset=off("m"))
        self.v = Buf(S, f32, device, fill=float("inf"), offset=off("v"))
        if valid:
            self.p.t[:valid] = torch.randn(valid, generator=g, device=device) * 0.02
            self.m.t[:valid] = torch.randn(valid, generator=g, device=device) * 1e-3
            self.v.t[:valid] = torch.randn(valid, generator=g, device=device).square() * 1e-6
        self.stride = S + stride_extra
        sd = torch.float32 if sdt == "f32" else torch.bfloat16
        self.sl = Buf(N * self.stride, sd, device, fill=float("nan"), offset=off("sl"))
        x = torch.randn(N, S, generator=g, device=device) * 1e-2
        self.sl.t.view(N, self.stride)[:, :S] = x.to(sd)
        if valid < S:
            self.sl.t.view(N, self.stride)[:, valid:S] = float("nan")   # pad garbage
        self.out = Buf(S, torch.bfloat16, device, fill=1.5, offset=off("out")) if bf16 else None
        self.gout = Buf(S, f32, device, fill=float("nan"), offset=off("gout")) if gout else None
        for b in self.bufs():
            b.seal()

    def bufs(self):
        return [b for b in (self.p, self.m, self.v, self.sl, self.out, self.gout) if b is not None]

    def snapshot(self):
        return (PR.f64(self.p.t), PR.f64(self.m.t), PR.f64(self.v.t),
                PR.widen_slices(self.sl.t.view(self.N, self.stride)[:, :self.S], self.sdt))

    def mt(self):
        return {"param_fp32": self.p.t, "exp_avg": self.m.t, "exp_avg_sq": self.v.t,
                "grad_slices": self.sl.t, "slice_stride": self.stride,
                "unshard_bf16_out": self.out.t if self.out else None,
                "grad_shard_out": self.gout.t if self.gout else None,
                "shard_numel": self.S, "valid": self.valid}

    def check(self, name, snap, t, check_g=True, hp=HP, widen=False):
        """``widen``: judge p' with the denominator term in its floor (the
        cases that draw 33 slices or a random slice count)."""
        p0, m0, v0, sl = snap
        ref = O.rank_step(p0, m0, v0, sl, self.valid, t, hp)
        va = self.valid
        fl = PR.floors(p0[:va], m0[:va], v0[:va], sl[:, :va], {k: r[:va] for k, r in ref.items()}, hp, t,
                       widen=widen)
        gp = self.p.t.cpu().numpy()
        PR.assert_close(f"{name} p", gp[:va], ref["p"][:va], fl["p"])
        PR.assert_close(f"{name} m", self.m.t.cpu().numpy()[:va], ref["m"][:va], fl["m"])
        PR.assert_close(f"{name} v", self.v.t.cpu().numpy()[:va], ref["v"][:va], fl["v"])
        for b, nm in ((self.p, "p"), (self.m, "m"), (self.v, "v")):
            PR.check_pad_zero(f"{name} {nm}", b.t.cpu().numpy(), va)
        if self.out is not None:
            bits = PR.bf16_bits(self.out.t)
            PR.check_bf16(f"{name} bf16", bits[:va], gp[:va], ref["p"][:va], fl["p"])
            PR.check_pad_zero(f"{name} bf16", bits, va)
        if self.gout is not None and check_g:
            gg = self.gout.t.cpu().numpy()
            PR.assert_close(f"{name} g", gg[:va], ref["g"][:va], fl["g"])
            PR.check_pad_zero(f"{name} g", gg, va)
        for b in self.bufs():
            b.check_guards(name)


SPECS = [  # (S, valid, offset, stride_extra)
    (0, 0, 0, 0),
    (1, 1, 0, 0),
    (7, 0, 0, 0),
    (8, 8, 0, 0),
    (2048 * 5 + 1237, 2048 * 5 + 1230, 0, 0),     # several tiles + ragged tail, partial pad
    (16384, 16384, 0, 40),                         # wider slice stride
    (9001, 8999, 1, 0),                            # misaligned: element path
    (4096, 3, 0, 0),                               # nearly all padding
    (70001, 70001, 0, 0),
    (256, 256, 0, 0),                              # exactly one workgroup tile
    (257, 255, 0, 0),                              # one tile and one element, partial group at valid
    (2048 + 256, 2048 + 252, 4, 0),                # bf16 buffers 8- but not 16-byte aligned: vector path
    (4096 + 1000, 4096 + 1000, 4, 4),              # the same with a wider stride that keeps slices aligned
    (4095, 4095, 0, 2),                            # stride that misaligns slice q > 0
    (5013, 5009, 1, 3),                            # every buffer 1 element past a vector boundary:
                                                   # split into a head of 3 and an aligned body
    (4099, 4099, 2, 1),                            # the same 2 elements past: head of 2
    (3001, 2990, 3, 3),                            # 3 past: head of 1
    (12, 7, 1, 0),                                 # just long enough to split (head + one group)
    (10, 6, 1, 2),                                 # one element too short: element path
]


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
# N outside 1, 2, 4, 8 reads its slices in batches (4 bf16 or 2 fp32 slices
# each): 5, 6, 7 and 33 end on every partial batch, 16 on whole ones.
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8, 16, 33])
def test_mt_step_parity(gpu, N, sdt):
    shards = [Shard(S, va, N, sdt, gpu, seed=100 * N + i, offset=o, stride_extra=x,
                    bf16=(i % 3 != 1), gout=(i % 2 == 0))
              for i, (S, va, o, x) in enumerate(SPECS)]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    info = plan.info()
    assert info["n_tensors"] == len(SPECS) and info["total_numel"] == sum(s[0] for s in SPECS)
    for t in (1, 2, 3):
        # fresh gradients each step; the state carries over (per-step resync)
        for i, s in enumerate(shards):
            g = torch.Generator(device=gpu)
            g.manual_seed(7 * t + i)
            x = torch.randn(N, s.S, generator=g, device=gpu) * 1e-2
            s.sl.t.view(N, s.stride)[:, :s.valid] = x[:, :s.valid].to(s.sl.t.dtype)
        snaps = [s.snapshot() for s in shards]
        plan.step(HP, t)
        torch.cuda.synchronize()
        for i, (s, snap) in enumerate(zip(shards, snaps)):
            s.check(f"N={N} {sdt} shard {i} t={t}", snap, t, widen=N == 33)
    plan.close()


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 6, 8, 33])
def test_single_calls_parity(gpu, N, sdt):
    for i, (S, va, o, x) in enumerate(SPECS):
        s = Shard(S, va, N, sdt, gpu, seed=1000 + i, offset=o, stride_extra=x)
        snap = s.snapshot()
        B.fsdp_reduce_grad_shard(s.gout.t, s.sl.t, sdt, s.stride, N, S, va)
        B.fsdp_adamw_shard_step(s.p.t, s.m.t, s.v.t, s.gout.t, S, va, HP, 1)
        B.fsdp_cast_unshard_bf16(s.out.t, s.p.t, S, va)
        torch.cuda.synchronize()
        s.check(f"single N={N} {sdt} case {i}", snap, 1, widen=N == 33)


@pytest.mark.parametrize("sdt,N", [("bf16", 8), ("f32", 4), ("f32", 3), ("bf16", 1), ("bf16", 7)])
def test_fused_equals_chain_bitwise(gpu, sdt, N):
    a = [Shard(S, va, N, sdt, gpu, seed=5000 + i, offset=o, stride_extra=x)
         for i, (S, va, o, x) in enumerate(SPECS)]
    b = [Shard(S, va, N, sdt, gpu, seed=5000 + i, offset=o, stride_extra=x)
         for i, (S, va, o, x) in enumerate(SPECS)]
    plan = B.MtPlan([s.mt() for s in a], N, sdt)
    for t in (1, 2):
        plan.step(HP, t)
        for s in b:
            B.fsdp_reduce_grad_shard(s.gout.t, s.sl.t, sdt, s.stride, N, s.S, s.valid)
            B.fsdp_adamw_shard_step(s.p.t, s.m.t, s.v.t, s.gout.t, s.S, s.valid, HP, t)
            B.fsdp_cast_unshard_bf16(s.out.t, s.p.t, s.S, s.valid)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(a, b)):
            for nm in ("p", "m", "v", "gout"):
                bx, by = getattr(x, nm).t, getattr(y, nm).t
                assert torch.equal(bx.view(torch.int32), by.view(torch.int32)), (i, nm, t)
            assert torch.equal(x.out.t.view(torch.int16), y.out.t.view(torch.int16)), (i, t)
    plan.close()


def test_deterministic_and_resumable(gpu):
    N, sdt = 8, "bf16"
    runs = []
    for _ in range(2):
        s = [Shard(S, va, N, sdt, gpu, seed=77 + i, offset=o, stride_extra=x)
             for i, (S, va, o, x) in enumerate(SPECS)]
        plan = B.MtPlan([x.mt() for x in s], N, sdt)
        for t in (1, 2, 3):
            plan.step(HP, t)
        torch.cuda.synchronize()
        runs.append([(x.p.t.clone(), x.m.t.clone(), x.v.t.clone(), x.out.t.clone()) for x in s])
        plan.close()
    for ra, rb in zip(*runs):
        for ta, tb in zip(ra, rb):
            assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))
    # checkpoint after step 1, reload into fresh buffers, continue: identical to uninterrupted
    s = [Shard(S, va, N, sdt, gpu, seed=77 + i, offset=o, stride_extra=x)
         for i, (S, va, o, x) in enumerate(SPECS)]
    plan = B.MtPlan([x.mt() for x in s], N, sdt)
    plan.step(HP, 1)
    torch.cuda.synchronize()
    ckpt = [(x.p.t.clone(), x.m.t.clone(), x.v.t.clone()) for x in s]
    plan.close()
    r = [Shard(S, va, N, sdt, gpu, seed=77 + i, offset=o, stride_extra=x)
         for i, (S, va, o, x) in enumerate(SPECS)]
    for x, (p, m, v) in zip(r, ckpt):
        x.p.t.copy_(p), x.m.t.copy_(m), x.v.t.copy_(v)
    plan = B.MtPlan([x.mt() for x in r], N, sdt)
    plan.step(HP, 2)
    plan.step(HP, 3)
    torch.cuda.synchronize()
    for x, (p, m, v, o) in zip(r, runs[0]):
        for ta, tb in ((x.p.t, p), (x.m.t, m), (x.v.t, v), (x.out.t, o)):
            assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))
    plan.close()


def test_nan_inf_propagate(gpu):
    N, sdt, S = 4, "f32", 4096
    s = Shard(S, S, N, sdt, gpu, seed=9)
    s.sl.t.view(N, S)[1, 100] = float("nan")
    s.sl.t.view(N, S)[2, 200] = float("inf")
    s.sl.t.view(N, S)[0, 300] = float("inf")
    s.sl.t.view(N, S)[3, 300] = float("-inf")
    snap = s.snapshot()
    plan = B.MtPlan([s.mt()], N, sdt)
    plan.step(HP, 1)
    torch.cuda.synchronize()
    s.check("nan/inf", snap, 1)
    p = s.p.t.cpu().numpy()
    assert np.isnan(p[[100, 200, 300]]).all() and np.isfinite(np.delete(p, [100, 200, 300])).all()
    bits = PR.bf16_bits(s.out.t)
    assert all((bits[i] & 0x7FFF) == 0x7FC0 for i in (100, 200, 300))
    plan.close()


def test_cast_rounding_classes(gpu):
    # every bf16 top half x the rounding-relevant low halves, plus random patterns
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    rng = np.random.default_rng(1)
    bits = np.concatenate([(hi[:, None] | lows[None, :]).ravel(),
                           rng.integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)])
    n = bits.size
    x = torch.from_numpy(bits.view(np.int32).copy()).to(gpu).view(torch.float32)
    out = torch.full((n,), 12345, dtype=torch.int16, device=gpu)
    B.fsdp_cast_unshard_bf16(out, x, n, n)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    f = bits.view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        ref = O.bf16_rne(f)
    assert np.array_equal(got, ref)


# Hyperparameters at the edges of their ranges: no step, no decay, no first or
# second moment memory, no epsilon, and step counts where both bias
# corrections have reached 1.
EDGE_HPARAMS = [
    ("lr 0", dict(HP, lr=0.0), 1),
    ("no weight decay", dict(HP, weight_decay=0.0), 2),
    ("beta1 0", dict(HP, beta1=0.0), 2),
    ("beta2 0", dict(HP, beta2=0.0), 2),
    ("eps 0", dict(HP, eps=0.0), 1),
    ("step 10000", HP, 10000),
    ("step 2^40", HP, 1 << 40),
    ("large lr and decay", dict(HP, lr=0.5, weight_decay=0.5), 3),
]


@pytest.mark.parametrize("name,hp,t", EDGE_HPARAMS, ids=[e[0] for e in EDGE_HPARAMS])
def test_hparam_edges(gpu, name, hp, t):
    N, sdt = 4, "bf16"
    shards = [Shard(S, va, N, sdt, gpu, seed=300 + i, offset=o, stride_extra=x)
              for i, (S, va, o, x) in enumerate(SPECS)]
    snaps = [s.snapshot() for s in shards]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    plan.step(hp, t)
    torch.cuda.synchronize()
    for i, (s, snap) in enumerate(zip(shards, snaps)):
        s.check(f"{name} shard {i}", snap, t, hp=hp)
        if hp["lr"] == 0.0:
            # no step at all: decay factor 1 and a zero update leave p's bits alone
            va = s.valid
            assert np.array_equal(s.p.t.cpu().numpy()[:va].view(np.uint32),
                                  snap[0][:va].astype(np.float32).view(np.uint32)), name
    plan.close()


def test_fp32_range_edges(gpu):
    """Where fp32's range, not its precision, decides the result.

    * Overflow: a mean gradient of about 1e30 has a square beyond fp32, so v'
      saturates to +inf, m'/(sqrt(v')+eps) is 0 and p' is exactly p*(1-lr*wd),
      as fp32 AdamW computes it (the float64 oracle keeps the square finite and
      is not the reference for these elements).
    * Subnormals: parameters, first moments and gradients in fp32's subnormal
      range, compared with the oracle with an absolute allowance of a few
      subnormal spacings (2**-149) on top of the relative bound.  The second
      moments stay normal: where eps alone bounds the denominator, the
      update multiplies a subnormal moment's absolute error by lr/eps, a
      property of fp32 arithmetic rather than of the kernel.
    """
    N, sdt, S = 4, "f32", 4096
    s = Shard(S, S, N, sdt, gpu, seed=21)
    sl = s.sl.t.view(N, S)
    big = slice(0, 256)
    sl[:, big] = 0.0
    sl[0, big] = torch.linspace(-1e30, 1e30, 256, device=gpu)
    sl[0, 128] = 3e30                                   # no exact zero in the group
    sub = slice(256, 512)                                # subnormal p and m, zero gradient
    sl[:, sub] = 0.0
    gen = torch.Generator(device=gpu)
    gen.manual_seed(3)
    s.p.t[sub] = torch.randn(256, generator=gen, device=gpu) * 1e-40
    s.m.t[sub] = torch.randn(256, generator=gen, device=gpu) * 1e-40
    s.v.t[sub] = torch.rand(256, generator=gen, device=gpu) * 1e-6 + 1e-7
    tiny = slice(512, 768)                               # subnormal gradients
    sl[:, tiny] = torch.randn(N, 256, generator=gen, device=gpu) * 1e-39
    snap = s.snapshot()
    plan = B.MtPlan([s.mt()], N, sdt)
    plan.step(HP, 1)
    torch.cuda.synchronize()
    p0, m0, v0, x = snap
    gp, gm, gv = (b.t.cpu().numpy() for b in (s.p, s.m, s.v))

    decay = np.float32(1.0 - HP["lr"] * HP["weight_decay"])
    assert np.all(np.isposinf(gv[big])), "v' of an overflowing square must be +inf"
    want = (p0[big].astype(np.float32) * decay).astype(np.float32)
    assert np.array_equal(gp[big].view(np.uint32), want.view(np.uint32)), "p' must be p*(1-lr*wd)"
    ref = O.rank_step(p0, m0, v0, x, S, 1, HP)
    fl = PR.floors(p0, m0, v0, x, ref, HP, 1)
    PR.assert_close("overflow m", gm[big], ref["m"][big], fl["m"][big])

    rest = np.r_[256:S]
    allowance = 4 * 2.0 ** -149
    for nm, got in (("p", gp), ("m", gm), ("v", gv)):
        PR.assert_close(f"range {nm}", got[rest], ref[nm][rest], fl[nm][rest], abs_tol=allowance)
    bits = PR.bf16_bits(s.out.t)
    assert np.array_equal(bits, O.bf16_rne(gp.astype(np.float64))), "bf16 is RNE of the fp32 result"
    plan.close()


@pytest.mark.parametrize("sdt,N", [("f32", 1), ("bf16", 3), ("bf16", 8), ("f32", 16), ("f32", 33)])
def test_fp32_replica_bit_exact(gpu, sdt, N):
    """Every element of the fused step equals the kernel's stated fp32
    sequence bit for bit, so any distance to the float64 oracle is the
    conditioning of fp32 arithmetic, not an error of the kernel."""
    shards = [Shard(S, va, N, sdt, gpu, seed=900 + i, offset=o, stride_extra=x)
              for i, (S, va, o, x) in enumerate(SPECS)]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    for t in (1, 2):
        snaps = [s.snapshot() for s in shards]
        plan.step(HP, t)
        torch.cuda.synchronize()
        for i, (s, (p0, m0, v0, x)) in enumerate(zip(shards, snaps)):
            va = s.valid
            if va == 0:
                continue
            rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, x, va, t, HP)
            for nm, got, want in (("p", s.p.t, rp), ("m", s.m.t, rm), ("v", s.v.t, rv)):
                g = got.cpu().numpy()[:va]
                bad = g.view(np.uint32) != want.view(np.uint32)
                assert not bad.any(), (f"N={N} {sdt} shard {i} t={t} {nm}: {bad.sum()} differ, "
                                       f"first {np.flatnonzero(bad)[:3]} got {g[bad][:3]} want {want[bad][:3]}")
    plan.close()


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("off,head", [(1, 3), (2, 2), (3, 1)])
def test_misaligned_shard_split_equals_element_path(gpu, sdt, off, head):
    """A shard whose fp32 buffers all start `off` elements past a vector
    boundary is split into a head of 4 - off elements and an aligned body
    (one more chunk entry): (a) with the slices in phase after the split,
    (b) with a slice stride that leaves them out of phase (the body reads them
    as shifted vectors).  (c) The same data with one moment buffer in another
    phase cannot be split and runs element by element.  All give identical
    bits."""
    N, S, va = 3, 5013, 5009
    a = Shard(S, va, N, sdt, gpu, seed=8100 + off, offset=off, stride_extra=3)   # stride % 4 == 0
    b = Shard(S, va, N, sdt, gpu, seed=8100 + off, offset=off, stride_extra=1)   # stride % 4 == 2
    c = Shard(S, va, N, sdt, gpu, seed=8100 + off, stride_extra=3,
              offset={"p": off, "m": (off + 1) % 4, "v": off, "sl": off, "out": off, "gout": off})
    plans = [B.MtPlan([x.mt()], N, sdt) for x in (a, b, c)]
    split = 1 + -(-(S - head) // 2048)
    assert [pl.info()["n_chunks"] for pl in plans] == [split, split, -(-S // 2048)]
    for t in (1, 2):
        snap = a.snapshot()
        for pl in plans:
            pl.step(HP, t)
        torch.cuda.synchronize()
        a.check(f"split off={off} {sdt} t={t}", snap, t)
        for y in (b, c):
            for nm in ("p", "m", "v", "gout"):
                assert torch.equal(getattr(a, nm).t.view(torch.int32), getattr(y, nm).t.view(torch.int32)), (nm, t)
            assert torch.equal(a.out.t.view(torch.int16), y.out.t.view(torch.int16)), t
        for x in (a, b, c):
            for bf in x.bufs():
                bf.check_guards(f"split off={off}")
    for pl in plans:
        pl.close()


# slices (per-slice phases through the stride) and bf16 copies at every
# element phase, with the fp32 state aligned: the vector path reads the
# slices as shifted vectors and stores the copies in narrower pieces
PLACEMENTS = [
    {"sl": 1, "out": 1}, {"sl": 2, "out": 2}, {"sl": 3, "out": 3},
    {"sl": 0, "out": 1}, {"sl": 1, "out": 0}, {"sl": 2, "out": 3},
]


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 8])
def test_misaligned_slices_and_copies_equal_aligned(gpu, N, sdt):
    """The same data with every buffer aligned, and with the slices and the
    bf16 copy at other element phases (strides in and out of phase): the
    fused step and the clipped step give identical bits, guards intact."""
    specs = [(2048 * 3 + 517, 2048 * 3 + 510, x) for x in (0, 1, 2, 3)] + [(300, 297, 2), (9, 9, 1)]
    # the reference: every buffer aligned, strides keeping every slice aligned
    mk = lambda pl, aligned: [Shard(S, va, N, sdt, gpu, seed=8300 + 10 * i + N, offset=pl,
                                    stride_extra=(-S) % 4 if aligned else x)
                              for i, (S, va, x) in enumerate(specs)]
    for pl in PLACEMENTS:
        a, b = mk({}, True), mk(pl, False)
        plan_a = B.MtPlan([s.mt() for s in a], N, sdt)
        plan_b = B.MtPlan([s.mt() for s in b], N, sdt)
        sq = [torch.zeros(1, dtype=torch.float64, device=gpu) for _ in range(2)]
        coef = [torch.zeros(1, dtype=torch.float32, device=gpu) for _ in range(2)]
        snaps = [s.snapshot() for s in b]
        for k, plan in enumerate((plan_a, plan_b)):
            plan.step(HP, 1)
        torch.cuda.synchronize()
        for i, (s, snap) in enumerate(zip(b, snaps)):
            s.check(f"placement {pl} N={N} {sdt} shard {i}", snap, 1)
        for k, plan in enumerate((plan_a, plan_b)):
            plan.reduce_sqnorm(sq[k])
            B.fsdp_clip_coef(coef[k], None, sq[k], 1, 0.05)
            plan.step_clipped(HP, 2, coef[k])
        torch.cuda.synchronize()
        assert sq[0].view(torch.int64).item() == sq[1].view(torch.int64).item()
        for i, (x, y) in enumerate(zip(a, b)):
            for nm in ("p", "m", "v", "gout"):
                assert torch.equal(getattr(x, nm).t.view(torch.int32), getattr(y, nm).t.view(torch.int32)), \
                    (pl, i, nm)
            assert torch.equal(x.out.t.view(torch.int16), y.out.t.view(torch.int16)), (pl, i)
            for bf in y.bufs():
                bf.check_guards(f"placement {pl} shard {i}")
        plan_a.close()
        plan_b.close()


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_single_calls_at_any_alignment_equal_aligned(gpu, sdt):
    """The three single-shard calls with the slices, the gradient the AdamW
    call reads and the bf16 copy off their vector boundaries (the fp32 state
    and the reduce's output aligned): identical bits to the all-aligned
    placement, guards intact."""
    N = 3
    S, va = 2048 * 2 + 333, 2048 * 2 + 330
    for pl in PLACEMENTS:
        a = Shard(S, va, N, sdt, gpu, seed=8500, stride_extra=(-S) % 4)
        b = Shard(S, va, N, sdt, gpu, seed=8500, offset=pl, stride_extra=1)
        grads = []
        for s, off in ((a, 0), (b, pl["sl"] or 1)):
            B.fsdp_reduce_grad_shard(s.gout.t, s.sl.t, sdt, s.stride, N, S, va)
            g = Buf(S, torch.float32, gpu, fill=float("nan"), offset=off)  # the gradient elsewhere
            g.t.copy_(s.gout.t)
            g.seal()
            grads.append(g)
            B.fsdp_adamw_shard_step(s.p.t, s.m.t, s.v.t, g.t, S, va, HP, 1)
            B.fsdp_cast_unshard_bf16(s.out.t, s.p.t, S, va)
        torch.cuda.synchronize()
        for nm in ("p", "m", "v", "gout"):
            assert torch.equal(getattr(a, nm).t.view(torch.int32), getattr(b, nm).t.view(torch.int32)), (pl, nm)
        assert torch.equal(a.out.t.view(torch.int16), b.out.t.view(torch.int16)), pl
        for bf in b.bufs() + grads:
            bf.check_guards(f"single calls {pl}")


# the largest slice count the ABI accepts, and one short of it (a partial
# last batch), on small ragged shards
MAX_N_SPECS = [(2048 + 300, 2048 + 297, 0, 0), (1001, 1001, 0, 3), (255, 250, 4, 1), (37, 37, 1, 3)]


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1023, 1024])
def test_max_slice_count(gpu, N, sdt):
    shards = [Shard(S, va, N, sdt, gpu, seed=7700 + i, offset=o, stride_extra=x)
              for i, (S, va, o, x) in enumerate(MAX_N_SPECS)]
    plan = B.MtPlan([s.mt() for s in shards], N, sdt)
    snaps = [s.snapshot() for s in shards]
    plan.step(HP, 1)
    torch.cuda.synchronize()
    for i, (s, snap) in enumerate(zip(shards, snaps)):
        s.check(f"N={N} {sdt} shard {i}", snap, 1)
        p0, m0, v0, x = snap
        rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, x, s.valid, 1, HP)
        for nm, got, want in (("p", s.p.t, rp), ("m", s.m.t, rm), ("v", s.v.t, rv)):
            assert np.array_equal(got.cpu().numpy()[:s.valid].view(np.uint32), want.view(np.uint32)), \
                f"N={N} {sdt} shard {i} {nm}: differs from the fp32 replica"
    plan.close()
    # the single-shard reduce of the same slices, bit for bit against their fp32 sum
    s = shards[0]
    B.fsdp_reduce_grad_shard(s.gout.t, s.sl.t, sdt, s.stride, N, s.S, s.valid)
    torch.cuda.synchronize()
    x = snaps[0][3]
    want = x[:, :s.valid].astype(np.float32)
    acc = want[0].copy()
    for q in range(1, N):
        acc = (acc + want[q]).astype(np.float32)
    acc = acc * np.float32(1.0 / N) if N & (N - 1) == 0 else acc / np.float32(N)
    assert np.array_equal(s.gout.t.cpu().numpy()[:s.valid].view(np.uint32), acc.astype(np.float32).view(np.uint32))
