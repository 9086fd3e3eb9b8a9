"""One shard of more than 2^32 elements (a FLAT unit of a 7B model at N = 1 or
2 is one such shard): 64-bit element offsets in the plan's chunk table and in
the single-shard kernels, past 2^31 and 2^32.

Step 1 runs through a multi-tensor plan (the fused kernel), step 2 through the
three single-shard calls on the same buffers.  Sampled elements (random ones,
windows around 2^31 and 2^32, and the ragged tail with its padding) are
checked against the float64 oracle within the fp32 tolerance and bit for bit
against the kernel's stated fp32 operation sequence.  About 95 GB of HBM.
"""

import numpy as np
import pytest
import torch

from oracle import step as O
from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS
from tests import parity as PR

pytestmark = pytest.mark.gpu

N = 2
S = (1 << 32) + 3 * 2048 + 517
VALID = S - 5


def _sample_index(rng):
    parts = [rng.integers(0, S, 1 << 20)]
    for edge in (1 << 31, 1 << 32):
        parts.append(np.arange(edge - 1024, edge + 1024))
    parts.append(np.arange(S - 3000, S))
    return np.unique(np.concatenate(parts))


def _fill_bf16(dst, gen, sigma, chunk=1 << 30):
    for a in range(0, dst.numel(), chunk):
        b = min(dst.numel(), a + chunk)
        dst[a:b] = (torch.randn(b - a, generator=gen, device=dst.device) * sigma).to(torch.bfloat16)


def _check(name, idx, before, after, t):
    p0, m0, v0, x = before
    p, m, v, g, out = after
    va = int(np.searchsorted(idx, VALID))        # sampled elements below valid come first
    ref = O.rank_step(p0, m0, v0, x, va, t, HPARAMS)
    fl = PR.floors(p0[:va], m0[:va], v0[:va], x[:, :va], {k: r[:va] for k, r in ref.items()},
                   HPARAMS, t)
    PR.assert_close(f"{name} g", g[:va], ref["g"][:va], fl["g"])
    PR.assert_close(f"{name} p", p[:va], ref["p"][:va], fl["p"])
    PR.assert_close(f"{name} m", m[:va], ref["m"][:va], fl["m"])
    PR.assert_close(f"{name} v", v[:va], ref["v"][:va], fl["v"])
    PR.check_bf16(f"{name} bf16", out[:va], p[:va], ref["p"][:va], fl["p"])
    rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, x, va, t, HPARAMS)
    for nm, got, want in (("p", p, rp), ("m", m, rm), ("v", v, rv)):
        bad = got[:va].view(np.uint32) != want.view(np.uint32)
        assert not bad.any(), f"{name} {nm}: {bad.sum()} sampled elements differ from the fp32 replica"
    for arr, nm in ((p, "p"), (m, "m"), (v, "v"), (g, "g"), (out, "bf16")):
        assert not np.any(arr[va:]), f"{name} {nm}: padding not +0"


def test_one_shard_beyond_2_pow_32_elements(gpu):
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(gpu)
    need = S * (3 * 4 + N * 2 + 2 + 4)
    if free < need + (8 << 30):
        pytest.skip(f"needs {need / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    print(f"one shard of {S:,} elements, valid {VALID:,}, N={N} bf16", flush=True)
    gen = torch.Generator(device=gpu)
    gen.manual_seed(2024)
    p = torch.empty(S, dtype=torch.float32, device=gpu)
    for a in range(0, S, 1 << 30):
        b = min(S, a + (1 << 30))
        p[a:b] = torch.randn(b - a, generator=gen, device=gpu) * 0.02
    m = torch.zeros(S, dtype=torch.float32, device=gpu)
    v = torch.zeros(S, dtype=torch.float32, device=gpu)
    sl = torch.empty((N, S), dtype=torch.bfloat16, device=gpu)
    for q in range(N):
        _fill_bf16(sl[q], gen, 1e-2)
    out = torch.full((S,), 12345, dtype=torch.int16, device=gpu)
    gout = torch.full((S,), float("nan"), dtype=torch.float32, device=gpu)
    idx_np = _sample_index(np.random.default_rng(5))
    idx = torch.from_numpy(idx_np).to(gpu)

    def snap():
        x = O.widen_bf16_bits(sl[:, idx].view(torch.int16).cpu().numpy().view(np.uint16))
        return PR.f64(p[idx]), PR.f64(m[idx]), PR.f64(v[idx]), x

    def result():
        return (p[idx].cpu().numpy(), m[idx].cpu().numpy(), v[idx].cpu().numpy(),
                gout[idx].cpu().numpy(), PR.bf16_bits(out[idx]))

    # step 1: the fused multi-tensor plan
    before = snap()
    plan = B.MtPlan([{"param_fp32": p, "exp_avg": m, "exp_avg_sq": v, "grad_slices": sl,
                      "slice_stride": S, "unshard_bf16_out": out, "grad_shard_out": gout,
                      "shard_numel": S, "valid": VALID}], N, "bf16")
    info = plan.info()
    assert info["total_numel"] == S and info["n_blocks"] == 8 * -(-S // 2048)
    plan.step(HPARAMS, 1)
    torch.cuda.synchronize()
    plan.close()
    _check("fused step 1", idx_np, before, result(), 1)

    # step 2: the three single-shard calls on the same buffers, fresh gradients
    for q in range(N):
        _fill_bf16(sl[q], gen, 1e-2)
    before = snap()
    B.fsdp_reduce_grad_shard(gout, sl, "bf16", S, N, S, VALID)
    B.fsdp_adamw_shard_step(p, m, v, gout, S, VALID, HPARAMS, 2)
    B.fsdp_cast_unshard_bf16(out, p, S, VALID)
    torch.cuda.synchronize()
    _check("single calls step 2", idx_np, before, result(), 2)

    del p, m, v, sl, out, gout, idx
    torch.cuda.empty_cache()
