"""A plan checks the further device buffers its calls take (a clip scale,
fp8 scales and amax arrays, a sum of squares) against its shards' own
buffers: an input may lie in the read-only gradient slices but not in a
buffer that some plan call writes, and an output may lie in none of them
(FSDP_E_ALIAS).  A refused call queues no work: every buffer of the plan is
unchanged after it.  The same calls with admissible placements run.

Two shards, N = 2 bf16 slices, every output present; shard 1 is one element
shorter (so a placement 8-byte aligned can straddle the end of its buffers)
and ragged (its slices are read in [0, valid) only, so their tail is no
buffer of the plan), and in the second plan it reads its slices through a
table of pointers to separate buffers.
"""

import pytest
import torch

from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS

pytestmark = pytest.mark.gpu

S, N = 1000, 2
SIZES = (S, S - 1)
VALID = (S, S - 100)


class Plan:
    def __init__(self, gpu, table):
        g = torch.Generator(device=gpu)
        g.manual_seed(4242)
        f32 = dict(dtype=torch.float32, device=gpu)
        # every array has a tail the plan does not name, so a placement that
        # straddles the end of a plan buffer stays inside the allocation
        self.p = torch.randn(2 * S + 64, generator=g, **f32) * 0.02
        self.m = torch.zeros(2 * S + 64, **f32)
        self.v = torch.zeros(2 * S + 64, **f32)
        self.gout = torch.zeros(2 * S + 64, **f32)
        self.out = torch.zeros(2 * S + 64, dtype=torch.int16, device=gpu)
        self.f8 = torch.zeros(2 * S + 64, dtype=torch.uint8, device=gpu)
        self.sl = (torch.randn(N, 2 * S, generator=g, device=gpu) * 1e-2).to(torch.bfloat16)
        self.tab = [self.sl[q, S:2 * S].clone() for q in range(N)] if table else None
        recs = []
        for i in range(2):
            o = i * S
            r = {"param_fp32": self.p.data_ptr() + 4 * o, "exp_avg": self.m.data_ptr() + 4 * o,
                 "exp_avg_sq": self.v.data_ptr() + 4 * o,
                 "grad_slices": self.sl.data_ptr() + 2 * o, "slice_stride": 2 * S,
                 "unshard_bf16_out": self.out.data_ptr() + 2 * o,
                 "grad_shard_out": self.gout.data_ptr() + 4 * o,
                 "unshard_fp8_out": self.f8.data_ptr() + o, "shard_numel": SIZES[i],
                 "valid": VALID[i]}
            if table and i == 1:
                r.pop("grad_slices")
                r.pop("slice_stride")
                r["grad_slice_ptrs"] = self.tab
            recs.append(r)
        self.plan = B.MtPlan(recs, N, "bf16")
        self.far = torch.zeros(64, **f32)

    def buffers(self):
        bs = [self.p, self.m, self.v, self.gout, self.out, self.f8, self.sl] + (self.tab or [])
        return [b.view(torch.uint8).clone() for b in bs]

    def places(self):
        """Named addresses and whether an input / an output may sit there."""
        sl_row1 = self.sl.data_ptr() + 2 * 2 * S
        pl = {
            "inside shard 1's param": (self.p.data_ptr() + 4 * (S + 10), False, False),
            "straddling the end of shard 1's grad_shard_out":
                (self.gout.data_ptr() + 4 * (S + SIZES[1] - 1), False, False),
            "inside shard 0's fp8 codes": (self.f8.data_ptr() + 40, False, False),
            "inside shard 0's bf16 copy": (self.out.data_ptr() + 64, False, False),
            "inside shard 0's slice 1": (sl_row1 + 2 * 20, True, False),
            "just past every plan buffer": (self.p.data_ptr() + 4 * 2 * S, True, True),
            "in a separate buffer": (self.far.data_ptr(), True, True),
        }
        if self.tab is None:
            # shard 1's slices are read in [0, valid): their tail is not the plan's
            pl["in the unread tail of shard 1's slice 1"] = (sl_row1 + 2 * (S + VALID[1] + 8), True, True)
        else:
            pl["inside shard 1's table slice 0"] = (self.tab[0].data_ptr() + 2 * 100, True, False)
        return pl

    def calls(self):
        """(name, is_output, function of an address) for every checked argument."""
        far, pl = self.far, self.plan
        return [
            ("sqnorm_out of fsdp_mt_reduce_sqnorm", True, lambda a: pl.reduce_sqnorm(a)),
            ("sqnorm_out of fsdp_mt_reduce_accumulate", True,
             lambda a: pl.reduce_accumulate(1, a)),
            ("grad_scale of fsdp_mt_step_clipped", False, lambda a: pl.step_clipped(HPARAMS, 2, a)),
            ("amax_out of fsdp_mt_step_amax", True, lambda a: pl.step_amax(HPARAMS, 3, a)),
            ("amax_ranks of fsdp_mt_cast_fp8", False, lambda a: pl.cast_fp8(a, 1, far[8:10])),
            ("scale_out of fsdp_mt_cast_fp8", True, lambda a: pl.cast_fp8(far[16:18], 1, a)),
            ("scale_in of fsdp_mt_step_fp8", False,
             lambda a: pl.step_fp8(HPARAMS, 4, a, far[24:26])),
            ("amax_out of fsdp_mt_step_fp8", True,
             lambda a: pl.step_fp8(HPARAMS, 4, far[32:34], a)),
        ]


@pytest.mark.parametrize("table", [False, True], ids=["stride", "table"])
def test_plan_call_buffers_checked_against_the_plan(gpu, table):
    P = Plan(gpu, table)
    P.far.fill_(1.0)
    P.plan.step(HPARAMS, 1)            # grad_shard_out holds a reduced gradient from here on
    torch.cuda.synchronize()
    refused = allowed = 0
    for place, (addr, ok_in, ok_out) in P.places().items():
        for name, is_out, call in P.calls():
            ok = ok_out if is_out else ok_in
            before = P.buffers()
            if ok:
                call(addr)
                torch.cuda.synchronize()
                allowed += 1
                continue
            with pytest.raises(B.FsdpError) as e:
                call(addr)
            assert e.value.name == "FSDP_E_ALIAS", f"{name} {place}: {e.value}"
            torch.cuda.synchronize()
            for i, (x, y) in enumerate(zip(before, P.buffers())):
                assert torch.equal(x, y), f"{name} {place}: refused call changed buffer {i}"
            refused += 1
    assert refused > 0 and allowed > 0
    P.plan.close()
