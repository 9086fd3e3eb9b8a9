"""Slices in N separate buffers (a table of slice pointers per shard) against
the same slices at one base and a stride.

The arithmetic is the same either way, so every output must be bit-identical:
the fused step, the clipped step (reduce with sum of squares, coefficient,
scaled update) and the one-pass fp8 step, on ragged shards, for N = 1, 3 and
8 in both slice dtypes.  Each slice buffer has its own offset: some keep the
vector alignment, some break it (the shard then takes the element path).
Plans mix shards of both forms, and the table's shards are also checked
against the oracle.  Guard words around every slice buffer must survive.
"""

import pytest
import torch

from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS
from tests.test_gpu_kernels import SPECS, Buf, Shard

pytestmark = pytest.mark.gpu


def _tabled(s, gpu, misalign, offset=None):
    """Copies of shard s's slices, one buffer each, and its plan record.
    ``offset``: every buffer that many elements past its allocation's start."""
    N, S = s.N, s.S
    dt = s.sl.t.dtype
    bufs = []
    for q in range(N):
        if offset is not None:
            off = offset
        else:
            off = (q * 3 + 1) % 5 if misalign else 4 * (q % 2)
        b = Buf(S, dt, s.p.t.device, fill=float("nan"), offset=off)
        b.t.copy_(s.sl.t.view(N, s.stride)[q, :S])
        b.seal()
        bufs.append(b)
    rec = s.mt()
    rec.pop("grad_slices")
    rec.pop("slice_stride")
    rec["grad_slice_ptrs"] = [b.t for b in bufs]
    return bufs, rec


def _outputs(shards):
    out = []
    for s in shards:
        for b in (s.p, s.m, s.v, s.out, s.gout):
            if b is not None:
                out.append(b.full.view(torch.int16).clone())
    return out


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 8])
def test_table_equals_stride_bitwise(gpu, N, sdt):
    mk = lambda: [Shard(S, va, N, sdt, gpu, seed=9000 + 10 * N + i, offset=o, stride_extra=x,
                        bf16=(i % 3 != 1), gout=True)
                  for i, (S, va, o, x) in enumerate(SPECS)]
    a, b = mk(), mk()
    # shards of b: even ones through a table (odd entries misaligned), odd ones as a stride
    tables, recs = [], []
    for i, s in enumerate(b):
        if i % 2 == 0:
            bufs, rec = _tabled(s, gpu, misalign=(i % 4 == 2))
            tables.append(bufs)
            recs.append(rec)
        else:
            recs.append(s.mt())
    n = len(SPECS)
    plan_a = B.MtPlan([s.mt() for s in a], N, sdt)
    plan_b = B.MtPlan(recs, N, sdt)
    del recs
    sq = [torch.zeros(1, dtype=torch.float64, device=gpu) for _ in range(2)]
    coef = [torch.zeros(1, dtype=torch.float32, device=gpu) for _ in range(2)]
    for k, plan in enumerate((plan_a, plan_b)):
        plan.step(HPARAMS, 1)
        plan.reduce_sqnorm(sq[k])
        B.fsdp_clip_coef(coef[k], None, sq[k], 1, 0.05)
        plan.step_clipped(HPARAMS, 2, coef[k])
    torch.cuda.synchronize()
    assert sq[0].view(torch.int64).item() == sq[1].view(torch.int64).item()
    assert coef[0].view(torch.int32).item() == coef[1].view(torch.int32).item()
    for i, (x, y) in enumerate(zip(_outputs(a), _outputs(b))):
        assert torch.equal(x, y), f"N={N} {sdt}: output {i} differs between the two forms"
    for bufs in tables:
        for buf in bufs:
            buf.check_guards("slice buffer")
    plan_a.close()
    plan_b.close()


def test_table_fp8_step_and_oracle(gpu):
    """The one-pass fp8 step through tables equals the stride form bit for
    bit (state, codes, amax), and the table's fused step matches the oracle."""
    N, sdt = 8, "bf16"
    mk = lambda: [Shard(S, va, N, sdt, gpu, seed=9500 + i, offset=o, stride_extra=x, gout=False)
                  for i, (S, va, o, x) in enumerate(SPECS)]
    a, b = mk(), mk()
    f8 = [[torch.full((max(s.S, 1),), 0xAB, dtype=torch.uint8, device=gpu)[:s.S] for s in st]
          for st in (a, b)]
    recs_b, tables = [], []
    for s, f in zip(b, f8[1]):
        bufs, rec = _tabled(s, gpu, misalign=False)
        tables.append(bufs)
        rec["unshard_fp8_out"] = f
        recs_b.append(rec)
    plan_a = B.MtPlan([dict(s.mt(), unshard_fp8_out=f) for s, f in zip(a, f8[0])], N, sdt)
    plan_b = B.MtPlan(recs_b, N, sdt)
    n = len(SPECS)
    scale = torch.full((n,), 448.0 / 0.05, dtype=torch.float32, device=gpu)
    amax = [torch.zeros(n, dtype=torch.float32, device=gpu) for _ in range(2)]
    snaps = [s.snapshot() for s in b]
    plan_a.step_fp8(HPARAMS, 1, scale, amax[0])
    plan_b.step_fp8(HPARAMS, 1, scale, amax[1])
    torch.cuda.synchronize()
    assert torch.equal(amax[0].view(torch.int32), amax[1].view(torch.int32))
    for x, y in zip(_outputs(a), _outputs(b)):
        assert torch.equal(x, y)
    for fa, fb in zip(f8[0], f8[1]):
        assert torch.equal(fa, fb)
    for i, (s, snap) in enumerate(zip(b, snaps)):
        s.check(f"table shard {i}", snap, 1, check_g=False)
    plan_a.close()
    plan_b.close()


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_table_shard_split_when_misaligned_alike(gpu, sdt):
    """Shards whose buffers, slice buffers included, all start 1-3 elements
    past a vector boundary are split into a short head and an aligned body
    in the table form too (the plan's copy of the table is shifted for the
    body): bit-identical to the same shards with their slices at a stride."""
    N = 5
    specs = [(5013, 5009, 1), (4099, 4099, 2), (3001, 2990, 3), (700, 700, 1)]
    mk = lambda: [Shard(S, va, N, sdt, gpu, seed=9700 + i, offset=o, stride_extra=(-S) % 4)
                  for i, (S, va, o) in enumerate(specs)]
    a, b = mk(), mk()
    tables, recs = [], []
    for (S, va, o), s in zip(specs, b):
        bufs, rec = _tabled(s, gpu, misalign=False, offset=o)
        tables.append(bufs)
        recs.append(rec)
    plan_a = B.MtPlan([s.mt() for s in a], N, sdt)
    plan_b = B.MtPlan(recs, N, sdt)
    del recs
    split_chunks = sum(1 + -(-(S - (4 - o)) // 2048) for S, va, o in specs)
    assert plan_a.info()["n_chunks"] == split_chunks
    assert plan_b.info()["n_chunks"] == split_chunks
    for t in (1, 2):
        snaps = [s.snapshot() for s in b]
        plan_a.step(HPARAMS, t)
        plan_b.step(HPARAMS, t)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(_outputs(a), _outputs(b))):
            assert torch.equal(x, y), f"{sdt} t={t}: output {i} differs between the two forms"
        for i, (s, snap) in enumerate(zip(b, snaps)):
            s.check(f"split table shard {i} t={t}", snap, t)
    for bufs in tables:
        for buf in bufs:
            buf.check_guards("slice buffer")
    plan_a.close()
    plan_b.close()
