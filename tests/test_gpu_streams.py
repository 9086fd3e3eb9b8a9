"""Plans are independent: two plans stepping at the same time on two streams
give bit for bit what they give one after the other.

Each plan runs a fused step, a clipped step (its sum-of-squares pass uses the
plan's own partial-sum buffer) and a one-pass fp8 step (its amax uses the
plan's own per-workgroup buffer) on ragged shards.  The concurrent run issues
the two plans' calls alternately on two streams of default priority, with no
ordering between the streams; every output is then compared with a
sequential run on fresh copies of the same inputs.
"""

import numpy as np
import pytest
import torch

from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS
from tests.test_gpu_kernels import SPECS, Shard

pytestmark = pytest.mark.gpu

N, SDT = 8, "bf16"


class PlanSet:
    def __init__(self, gpu, seed):
        self.shards = [Shard(S, va, N, SDT, gpu, seed=seed + i, offset=o, stride_extra=x,
                             bf16=(i % 2 == 0), gout=True)
                       for i, (S, va, o, x) in enumerate(SPECS)]
        self.f8 = [torch.full((max(s.S, 1),), 0xAB, dtype=torch.uint8, device=gpu)[:s.S]
                   for s in self.shards]
        n = len(self.shards)
        self.plan = B.MtPlan([dict(s.mt(), unshard_fp8_out=f) for s, f in zip(self.shards, self.f8)],
                             N, SDT)
        self.sq = torch.zeros(1, dtype=torch.float64, device=gpu)
        self.coef = torch.zeros(1, dtype=torch.float32, device=gpu)
        self.scale = torch.full((n,), 448.0 / 0.05, dtype=torch.float32, device=gpu)
        self.amax = torch.zeros(n, dtype=torch.float32, device=gpu)

    def ops(self, stream):
        """The calls of three steps, one closure per call, all on `stream`."""
        h = stream.cuda_stream
        return [
            lambda: self.plan.step(HPARAMS, 1, h),
            lambda: self.plan.reduce_sqnorm(self.sq, h),
            lambda: B.fsdp_clip_coef(self.coef, None, self.sq, 1, 0.05, h),
            lambda: self.plan.step_clipped(HPARAMS, 2, self.coef, h),
            lambda: self.plan.step_fp8(HPARAMS, 3, self.scale, self.amax, h),
        ]

    def outputs(self):
        out = []
        for s, f in zip(self.shards, self.f8):
            for b in s.bufs():
                out.append(b.full.view(torch.int16).cpu().numpy().copy())
            out.append(f.cpu().numpy().copy())
        for t in (self.sq, self.coef, self.amax):
            out.append(t.view(torch.int32).cpu().numpy().copy())
        return out

    def close(self):
        self.plan.close()


def test_two_plans_on_two_streams(gpu):
    # sequential reference
    a, b = PlanSet(gpu, 100), PlanSet(gpu, 200)
    default = torch.cuda.current_stream(gpu)
    for op in a.ops(default) + b.ops(default):
        op()
    torch.cuda.synchronize()
    ref_a, ref_b = a.outputs(), b.outputs()
    a.close()
    b.close()
    # concurrent: fresh copies, calls interleaved across two streams
    a, b = PlanSet(gpu, 100), PlanSet(gpu, 200)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=gpu), torch.cuda.Stream(device=gpu)
    for op_a, op_b in zip(a.ops(s1), b.ops(s2)):
        op_a()
        op_b()
    torch.cuda.synchronize()
    for name, ref, got in (("plan a", ref_a, a.outputs()), ("plan b", ref_b, b.outputs())):
        assert len(ref) == len(got)
        for i, (x, y) in enumerate(zip(ref, got)):
            assert np.array_equal(x, y), f"{name}: output {i} differs from the sequential run"
    a.close()
    b.close()


def _sleep_cycles_per_ms(gpu):
    """Rate of torch.cuda._sleep's counter, measured (its clock is the
    device's, not fixed)."""
    s = torch.cuda.current_stream(gpu)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)          # first launch outside the measurement
    e0.record(s)
    torch.cuda._sleep(1_000_000)
    e1.record(s)
    torch.cuda.synchronize()
    return 1_000_000 / max(e0.elapsed_time(e1), 1e-3)


def test_destroy_waits_for_its_plan_only(gpu):
    """fsdp_mt_plan_destroy returns once the plan's last launch has finished
    and waits for nothing else: a step queued on one stream behind a 100 ms
    delay has finished when destroy returns, while a 1.5 s delay on another
    stream, queued first, is still running."""
    import time

    rate = _sleep_cycles_per_ms(gpu)
    a = PlanSet(gpu, 300)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=gpu), torch.cuda.Stream(device=gpu)
    e_step, e_other = torch.cuda.Event(), torch.cuda.Event()
    with torch.cuda.stream(s2):
        torch.cuda._sleep(int(1500 * rate))
        e_other.record(s2)
    with torch.cuda.stream(s1):
        torch.cuda._sleep(int(100 * rate))
    a.plan.step(HPARAMS, 1, s1.cuda_stream)
    e_step.record(s1)
    t0 = time.perf_counter()
    a.close()
    waited = time.perf_counter() - t0
    step_done, other_done = e_step.query(), e_other.query()
    torch.cuda.synchronize()
    assert step_done, "destroy returned before the plan's step had finished"
    assert not other_done, f"destroy waited for another stream's work ({waited:.3f} s)"
    assert waited < 1.2, waited
