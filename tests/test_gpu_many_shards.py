"""A plan over 20,000 small ragged shards (an unwrapped model with many
parameters): the chunk and descriptor tables at scale, the per-shard
padding, and the per-shard amax of the fp8 path (one workgroup per shard).

Every shard is carved out of a few large buffers, a random gap after its
neighbour, so shards start at arbitrary element offsets: about a quarter of
them are aligned for the vector path.  In the rest every buffer starts the
same 1-3 elements past a vector boundary (the slice stride is a multiple of
4), so the plan splits each into a short element-path head and an aligned
body under one index; their amax must still be the shard's.  The gaps hold
guard values that must survive.  The oracle runs once over all
valid elements, since every shard shares the step's hyperparameters, and
each shard's padding must come out +0.
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from oracle import step as O
from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS
from tests import parity as PR

pytestmark = pytest.mark.gpu

N_SHARDS = 20_000
N, SDT = 3, "bf16"


def _layout(rng):
    sizes = rng.integers(0, 500, N_SHARDS)
    sizes[rng.random(N_SHARDS) < 0.02] = 0
    valid = np.where(rng.random(N_SHARDS) < 0.7, sizes,
                     (rng.random(N_SHARDS) * (sizes + 1)).astype(np.int64))
    gaps = rng.choice([4, 5, 6, 7, 8], N_SHARDS)
    offs = np.concatenate([[0], np.cumsum(sizes + gaps)[:-1]]) + 8
    total = int(offs[-1] + sizes[-1] + 64)
    total += (-total) % 4              # slices of one shard share their phase
    return sizes, valid, offs, total


def test_twenty_thousand_shards(gpu):
    rng = np.random.default_rng(77)
    sizes, valid, offs, total = _layout(rng)
    print(f"{N_SHARDS} shards, {int(sizes.sum()):,} elements, {int(valid.sum()):,} valid", flush=True)
    g = torch.Generator(device=gpu)
    g.manual_seed(78)
    f32 = dict(dtype=torch.float32, device=gpu)
    guard = -7.0e33
    p = torch.full((total,), guard, **f32)
    m = torch.full((total,), guard, **f32)
    v = torch.full((total,), guard, **f32)
    gout = torch.full((total,), guard, **f32)
    out = torch.full((total,), 12345, dtype=torch.int16, device=gpu)
    f8 = torch.full((total,), 0xAB, dtype=torch.uint8, device=gpu)
    sl = torch.full((N, total), 1.5, dtype=torch.bfloat16, device=gpu)
    # data in each shard's valid part, garbage in its padding
    mask = np.zeros(total, dtype=bool)
    inside = np.zeros(total, dtype=bool)
    for o, s, va in zip(offs, sizes, valid):
        mask[o:o + va] = True
        inside[o:o + s] = True
    mk = torch.from_numpy(mask).to(gpu)
    ins = torch.from_numpy(inside).to(gpu)
    pad = ins & ~mk
    p[mk] = torch.randn(int(mask.sum()), generator=g, device=gpu) * 0.02
    m[mk] = torch.randn(int(mask.sum()), generator=g, device=gpu) * 1e-3
    v[mk] = torch.randn(int(mask.sum()), generator=g, device=gpu).square() * 1e-6
    p[pad], m[pad], v[pad] = 1.0e30, float("nan"), float("inf")
    for q in range(N):
        sl[q][mk] = (torch.randn(int(mask.sum()), generator=g, device=gpu) * 1e-2).to(torch.bfloat16)
        sl[q][pad] = float("nan")
    recs = []
    es4, es2 = 4, 2
    for o, s, va in zip(offs.tolist(), sizes.tolist(), valid.tolist()):
        recs.append({"param_fp32": p.data_ptr() + es4 * o, "exp_avg": m.data_ptr() + es4 * o,
                     "exp_avg_sq": v.data_ptr() + es4 * o, "grad_slices": sl.data_ptr() + es2 * o,
                     "slice_stride": total, "unshard_bf16_out": out.data_ptr() + es2 * o,
                     "grad_shard_out": gout.data_ptr() + es4 * o,
                     "unshard_fp8_out": f8.data_ptr() + o, "shard_numel": s, "valid": va})
    plan = B.MtPlan(recs, N, SDT)
    info = plan.info()
    assert info["n_tensors"] == N_SHARDS and info["total_numel"] == int(sizes.sum())
    # a shard 1-3 elements past a boundary splits when its body keeps a group
    head = (4 - offs % 4) % 4
    split = (head > 0) & (valid >= head + 4)
    entries = np.where(split, 1 + -(-(sizes - head) // 2048), -(-sizes // 2048))
    assert info["n_chunks"] == int(entries.sum()), (info["n_chunks"], int(entries.sum()))
    print(f"{int(split.sum())} shards split into head and body", flush=True)

    p0, m0, v0 = PR.f64(p[mk]), PR.f64(m[mk]), PR.f64(v[mk])
    x = PR.widen_slices(sl[:, mk], SDT)
    scale = torch.from_numpy(
        (np.float32(448.0) / rng.uniform(0.01, 0.2, N_SHARDS)).astype(np.float32)).to(gpu)
    amax = torch.full((N_SHARDS,), -1.0, **f32)
    plan.step_fp8(HPARAMS, 1, scale, amax)
    torch.cuda.synchronize()

    ref = O.rank_step(p0, m0, v0, x, p0.size, 1, HPARAMS)
    fl = PR.floors(p0, m0, v0, x, ref, HPARAMS, 1)
    gp = p[mk].cpu().numpy()
    PR.assert_close("many p", gp, ref["p"], fl["p"])
    PR.assert_close("many m", m[mk].cpu().numpy(), ref["m"], fl["m"])
    PR.assert_close("many v", v[mk].cpu().numpy(), ref["v"], fl["v"])
    PR.assert_close("many g", gout[mk].cpu().numpy(), ref["g"], fl["g"])
    PR.check_bf16("many bf16", PR.bf16_bits(out[mk]), gp, ref["p"], fl["p"])
    # padding +0 everywhere, guards untouched outside the shards
    for name, t in (("p", p), ("m", m), ("v", v), ("g", gout)):
        assert torch.all(t[pad].view(torch.int32) == 0), f"{name}: padding not +0"
        assert torch.all(t[~ins] == guard), f"{name}: guard overwritten"
    assert torch.all(out[pad] == 0) and torch.all(out[~ins] == 12345)
    assert torch.all(f8[pad] == 0) and torch.all(f8[~ins] == 0xAB)
    # per-shard amax (fp32 bits) and codes of the GPU's own p'
    p_all = p.cpu().numpy()
    codes = f8.cpu().numpy()
    am = amax.cpu().numpy()
    sc = scale.cpu().numpy()
    for i, (o, s, va) in enumerate(zip(offs, sizes, valid)):
        seg = p_all[o:o + va]
        want = np.float32(np.abs(seg).max()) if va else np.float32(0.0)
        assert am[i].view(np.uint32) == want.view(np.uint32), (i, am[i], want)
        if i % 97 == 0:
            assert np.array_equal(codes[o:o + va], F.quantize(seg, sc[i])), i
    plan.close()
