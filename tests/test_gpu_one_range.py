"""GPU: the fused step of a plan whose shards lie back to back, run as one range.

fsdp_mt_step takes such a plan (every buffer contiguous from shard to shard,
every shard but the last unpadded, all on the plain vector path, and the
shards that start off a 2048-element chunk-entry boundary holding at most
1/256 of the elements) as one range from the kernel's arguments instead of
through the chunk table.  These tests check which
plans qualify (the plan's info reports it) and that the one-range step is
bit-identical to the table's on the same buffers, and within the oracle's
tolerance, for the three store policies.  The table side runs the same
shards listed in reverse order, which no longer lie back to back in list
order.
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
GUARD = 512
CHUNK = 2048


class Packed:
    """Shards of the given (shard_numel, valid) sizes back to back in one set of
    buffers, each buffer with guard words on both sides.  ``gap`` inserts that
    many elements before shard ``gap_at`` in every buffer; ``bf16_off`` shifts
    the bf16 copy by whole elements."""

    def __init__(self, sizes, N, sdt, dev, seed, bf16=True, gout=True, gap=0, gap_at=1,
                 bf16_off=0, gout_on=None):
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.sizes, self.N, self.sdt, self.dev = sizes, N, sdt, dev
        self.offs = []
        o = 0
        for i, (S, _) in enumerate(sizes):
            if i == gap_at:
                o += gap
            self.offs.append(o)
            o += S
        self.total = o
        # slice rows keep their vector alignment (a row start off it takes the
        # any-alignment loads, which the one-range step does not run)
        self.stride = (self.total + 63) // 64 * 64 + 256 if N > 1 else self.total
        f32 = torch.float32
        sd = torch.float32 if sdt == "f32" else torch.bfloat16

        def buf(n, dt, fill):
            full = torch.full((n + 2 * GUARD,), fill, dtype=dt, device=dev)
            return full, full[GUARD:GUARD + n]

        self.p_full, self.p = buf(self.total, f32, 1.0e30)
        self.m_full, self.m = buf(self.total, f32, float("nan"))
        self.v_full, self.v = buf(self.total, f32, float("inf"))
        self.sl_full, sl = buf(N * self.stride, sd, float("nan"))
        self.sl = sl.view(N, self.stride)
        for (S, va), off in zip(sizes, self.offs):
            if va:
                self.p[off:off + va] = torch.randn(va, generator=g, device=dev) * 0.02
                self.m[off:off + va] = torch.randn(va, generator=g, device=dev) * 1e-3
                self.v[off:off + va] = torch.randn(va, generator=g, device=dev).square() * 1e-6
                self.sl[:, off:off + va] = (torch.randn(N, va, generator=g, device=dev) * 1e-2).to(sd)
        self.out_full, self.out = (None, None)
        if bf16:
            self.out_full, out = buf(self.total + bf16_off, torch.bfloat16, 1.5)
            self.out = out[bf16_off:]
        self.gout_full, self.gout = buf(self.total, f32, float("nan")) if gout else (None, None)
        self.gout_on = gout_on
        self.fulls = [x for x in (self.p_full, self.m_full, self.v_full, self.sl_full, self.out_full,
                                  self.gout_full) if x is not None]
        self.guards = [torch.cat([x[:GUARD], x[-GUARD:]]).clone() for x in self.fulls]

    def records(self, order=None):
        recs = []
        for i in (order if order is not None else range(len(self.sizes))):
            (S, va), off = self.sizes[i], self.offs[i]
            with_g = self.gout is not None and (self.gout_on is None or i in self.gout_on)
            recs.append({
                "param_fp32": self.p[off:], "exp_avg": self.m[off:], "exp_avg_sq": self.v[off:],
                "grad_slices": self.sl.reshape(-1)[off:], "slice_stride": self.stride,
                "unshard_bf16_out": self.out[off:] if self.out is not None else None,
                "grad_shard_out": self.gout[off:] if with_g else None,
                "shard_numel": S, "valid": va})
        return recs

    def plan(self, order=None):
        return B.MtPlan(self.records(order), self.N, self.sdt)

    def state(self):
        return [x.clone() for x in (self.p, self.m, self.v)]

    def restore(self, st):
        for dst, src in zip((self.p, self.m, self.v), st):
            dst.copy_(src)

    def outputs(self):
        xs = [self.p, self.m, self.v] + [x for x in (self.out, self.gout) if x is not None]
        return [x.clone() for x in xs]

    def check_guards(self):
        for x, g in zip(self.fulls, self.guards):
            now = torch.cat([x[:GUARD], x[-GUARD:]])
            a = now.view(torch.int16) if now.dtype == torch.bfloat16 else now.view(torch.int32)
            b = g.view(torch.int16) if g.dtype == torch.bfloat16 else g.view(torch.int32)
            assert torch.equal(a, b), "guard words overwritten"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _info(pk, order=None):
    plan = pk.plan(order)
    try:
        return plan.info()
    finally:
        plan.close()


def _oracle_check(pk, snap, t, name):
    """Every shard against the oracle from the state before the step."""
    p0, m0, v0 = (PR.f64(x) for x in snap)
    sl = PR.widen_slices(pk.sl[:, :pk.total], pk.sdt)
    gp = pk.p.cpu().numpy()
    gm = pk.m.cpu().numpy()
    gv = pk.v.cpu().numpy()
    for (S, va), off in zip(pk.sizes, pk.offs):
        r = slice(off, off + va)
        ref = O.rank_step(p0[r], m0[r], v0[r], sl[:, r], va, t, HP)
        fl = PR.floors(p0[r], m0[r], v0[r], sl[:, r], ref, HP, t)
        PR.assert_close(f"{name} p@{off}", gp[r], ref["p"], fl["p"])
        PR.assert_close(f"{name} m@{off}", gm[r], ref["m"], fl["m"])
        PR.assert_close(f"{name} v@{off}", gv[r], ref["v"], fl["v"])
        for arr in (gp, gm, gv):
            PR.check_pad_zero(f"{name} pad@{off}", arr[off:off + S], va)
        if pk.out is not None:
            bits = PR.bf16_bits(pk.out[off:off + S])
            PR.check_bf16(f"{name} bf16@{off}", bits[:va], gp[r], ref["p"], fl["p"])
            PR.check_pad_zero(f"{name} bf16 pad@{off}", bits, va)
        if pk.gout is not None:
            PR.assert_close(f"{name} g@{off}", pk.gout[off:off + va].cpu().numpy(), ref["g"], fl["g"])


# (sizes, N, slice dtype, bf16 copy, stored gradient, expected store policy)
CASES = {
    "bf16_n8_wt": ([(3 * CHUNK, 3 * CHUNK), (CHUNK, CHUNK), (8 * CHUNK, 8 * CHUNK), (1003, 997)],
                   8, "bf16", True, True, 1),
    "f32_n1_ntwt": ([(5 * CHUNK, 5 * CHUNK), (2 * CHUNK, 2 * CHUNK), (CHUNK + 516, CHUNK + 513)],
                    1, "f32", True, False, 2),
    # 24 bytes read against 16 written: the tie, non-temporal write-through
    "f32_n3_runtime": ([(2 * CHUNK, 2 * CHUNK), (4 * CHUNK, 4 * CHUNK), (777, 777)],
                       3, "f32", False, True, 2),
    "bf16_n2_single": ([(6 * CHUNK + 260, 6 * CHUNK + 259)], 2, "bf16", True, False, 2),
    # a short shard whose successor starts off a chunk-entry boundary
    "bf16_n4_redealt": ([(256 * CHUNK, 256 * CHUNK), (512, 512), (508, 505)], 4, "bf16", True, True, 2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_one_range_bit_identical_to_the_table(case):
    sizes, N, sdt, bf16, gout, pol = CASES[case]
    dev = torch.device("cuda:0")
    pk = Packed(sizes, N, sdt, dev, seed=100 + sorted(CASES).index(case), bf16=bf16, gout=gout)
    rev = list(range(len(sizes)))[::-1]
    run_plan = pk.plan()
    table_plan = pk.plan(rev)
    try:
        ri, ti = run_plan.info(), table_plan.info()
        assert ri["step_one_range"] == 1, ri
        assert ti["step_one_range"] == (1 if len(sizes) == 1 else 0), ti
        assert ri["store_policy"] == pol and ti["store_policy"] == pol
        for t in (1, 2, 3):
            snap = pk.state()
            run_plan.step(HP, t)
            torch.cuda.synchronize()
            got = pk.outputs()
            _oracle_check(pk, snap, t, f"{case} t={t}")
            pk.restore(snap)
            table_plan.step(HP, t)
            torch.cuda.synchronize()
            want = pk.outputs()
            for a, b in zip(got, want):
                assert torch.equal(_bits(a), _bits(b)), f"{case} t={t}: one range differs from the table"
            pk.check_guards()
    finally:
        run_plan.close()
        table_plan.close()


def test_which_plans_run_as_one_range():
    dev = torch.device("cuda:0")
    whole = [(2 * CHUNK, 2 * CHUNK), (CHUNK, CHUNK), (300, 299)]
    assert _info(Packed(whole, 4, "bf16", dev, 1))["step_one_range"] == 1
    assert _info(Packed(whole, 4, "bf16", dev, 1), order=[1, 0, 2])["step_one_range"] == 0
    # a non-last shard that is whole tiles but not whole chunk entries, its
    # successor (almost half the elements) dealt off the table's XCDs
    assert _info(Packed([(CHUNK + 256, CHUNK + 256), (CHUNK, CHUNK)], 4, "bf16", dev, 2))["step_one_range"] == 0
    # shards off a chunk-entry boundary: 512 of 526,336 elements (at most
    # 1/256) run as one range, 2,560 of 526,332 do not
    big = 255 * CHUNK + 1536
    assert _info(Packed([(big, big), (512, 512), (CHUNK, CHUNK)], 2, "f32", dev, 10))["step_one_range"] == 1
    assert _info(Packed([(big - 4, big - 4), (512, 512), (CHUNK, CHUNK)], 2, "f32", dev, 11))["step_one_range"] == 0
    # padding in a non-last shard
    assert _info(Packed([(CHUNK, CHUNK - 1), (CHUNK, CHUNK)], 4, "bf16", dev, 3))["step_one_range"] == 0
    # a gap between two shards
    assert _info(Packed(whole, 4, "bf16", dev, 4, gap=CHUNK))["step_one_range"] == 0
    # a stored gradient on some shards only
    assert _info(Packed(whole, 4, "bf16", dev, 5, gout_on={0, 2}))["step_one_range"] == 0
    # a bf16 copy off its vector alignment (the any-alignment stores)
    assert _info(Packed(whole, 4, "bf16", dev, 6, bf16_off=1))["step_one_range"] == 0
    # slice rows off their vector alignment (the any-alignment loads)
    pk = Packed(whole, 4, "bf16", dev, 9)
    pk.stride += 1
    assert _info(pk)["step_one_range"] == 0
    # one shard of any length on the vector path
    assert _info(Packed([(1000, 990)], 8, "bf16", dev, 7))["step_one_range"] == 1
    # a plan with empty shards between full ones still lies back to back
    assert _info(Packed([(CHUNK, CHUNK), (0, 0), (CHUNK, CHUNK)], 2, "f32", dev, 8))["step_one_range"] == 1
