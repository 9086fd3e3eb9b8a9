"""fsdp_reduce_sqnorm_noalloc (the entry point that allocates no device memory)
against the entry point it varies, fsdp_mt_reduce_sqnorm on a plan that holds
the one shard, through the C ABI, on consecutive calls that reuse the
library's scratch array:

* the largest shard it accepts (N = 8 bf16 slices, a ragged tail), then a
  smaller one (N = 4 fp32 slices at an odd stride, so the shifted loads run),
  then one with a slice count that is not compiled in (N = 3): the reduced
  gradient and the fp64 sum of squares bit for bit equal to the plan call's,
  the padding +0, and both against the oracle (the mean of the slices within
  the mixed tolerance, the sum of squares within the fp64 summation bound);
* an empty shard writes 0; a shard one element past the limit is refused
  with FSDP_E_CAPACITY and queues nothing.
"""

import math

import numpy as np
import pytest
import torch

from oracle import clip as C
from oracle import step as O
from rank_step_amd import binding as B
from tests import parity as PR

pytestmark = pytest.mark.gpu

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _slices(dev, seed, n, S, stride, dtype):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    buf = torch.full((n * stride,), float("nan"), dtype=_DT[dtype], device=dev)
    x = torch.randn(n, S, generator=g, device=dev) * 1e-3
    for q in range(n):
        buf[q * stride:q * stride + S].copy_(x[q])
    return buf


def _plan_call(dev, sl, dtype, stride, n, S, valid):
    """The existing entry point: a one-shard plan's fsdp_mt_reduce_sqnorm."""
    z = [torch.zeros(S, device=dev) for _ in range(3)]
    g = torch.full((S,), float("nan"), device=dev)
    sq = torch.full((1,), float("nan"), dtype=torch.float64, device=dev)
    with B.MtPlan([{"param_fp32": z[0], "exp_avg": z[1], "exp_avg_sq": z[2], "grad_slices": sl,
                    "slice_stride": stride, "grad_shard_out": g, "shard_numel": S,
                    "valid": valid}], n, dtype) as plan:
        plan.reduce_sqnorm(sq)
        torch.cuda.synchronize()
    return g, sq


def _check_case(dev, seed, n, dtype, S, valid, stride):
    print(f"noalloc case: N={n} {dtype} S={S} valid={valid} stride={stride}", flush=True)
    sl = _slices(dev, seed, n, S, stride, dtype)
    g = torch.full((S,), float("nan"), device=dev)
    sq = torch.full((1,), float("nan"), dtype=torch.float64, device=dev)
    B.fsdp_reduce_sqnorm_noalloc(g, sq, sl, dtype, stride, n, S, valid)
    torch.cuda.synchronize()
    g_ref, sq_ref = _plan_call(dev, sl, dtype, stride, n, S, valid)
    gb = g.cpu().numpy().view(np.uint32)
    rb = g_ref.cpu().numpy().view(np.uint32)
    assert np.array_equal(gb, rb), f"{np.count_nonzero(gb != rb)} gradient words differ from the plan call"
    assert sq.cpu().numpy().view(np.uint64)[0] == sq_ref.cpu().numpy().view(np.uint64)[0], \
        (float(sq.item()), float(sq_ref.item()))
    assert np.all(gb[valid:] == 0), "padding not +0"
    # against the oracle: the mean of the slices, and the sum of squares of
    # the stored gradient within the fp64 bound for summing n_terms
    # non-negative terms, (n_terms - 1) * 2**-53 of their sum
    if dtype == "bf16":
        raw = sl.view(torch.int16).cpu().numpy().view(np.uint16)
        x = np.stack([O.widen_bf16_bits(raw[q * stride:q * stride + valid]) for q in range(n)])
    else:
        raw = sl.cpu().numpy()
        x = np.stack([raw[q * stride:q * stride + valid].astype(np.float64) for q in range(n)])
    gv = g.cpu().numpy()[:valid].astype(np.float64)
    PR.assert_close(f"noalloc N={n} g", gv, O.reduce_mean(x), np.mean(np.abs(x), axis=0))
    want = C.sq_norm(gv)
    got = float(sq.item())
    assert abs(got - want) <= max(valid - 1, 0) * 2.0 ** -53 * want, (got, want)
    del sl, x


def test_noalloc_consecutive_calls_match_plan_call(gpu):
    S = B.NOALLOC_MAX_NUMEL
    _check_case(gpu, 11, 8, "bf16", S, S - 5, S)                 # the largest shard
    _check_case(gpu, 12, 4, "f32", 300_001, 299_990, 300_003)    # smaller; odd slice stride
    _check_case(gpu, 13, 3, "bf16", 70_000, 70_000, 70_000)      # runtime slice count


def test_noalloc_empty_and_too_large(gpu):
    sq = torch.full((1,), float("nan"), dtype=torch.float64, device=gpu)
    sl = torch.zeros(8, dtype=torch.bfloat16, device=gpu)
    B.fsdp_reduce_sqnorm_noalloc(None, sq, sl, "bf16", 0, 1, 0, 0)
    torch.cuda.synchronize()
    assert float(sq.item()) == 0.0
    big = B.NOALLOC_MAX_NUMEL + 1
    g = torch.full((4,), 7.0, device=gpu)
    sq.fill_(-1.0)
    with pytest.raises(B.FsdpError) as e:
        # addresses that are never touched: the size is refused first
        B.fsdp_reduce_sqnorm_noalloc(g.data_ptr(), sq, sl.data_ptr(), "bf16", big, 1, big, big)
    assert e.value.name == "FSDP_E_CAPACITY" and "FSDP_NOALLOC_MAX_NUMEL" in str(e.value)
    torch.cuda.synchronize()
    assert float(sq.item()) == -1.0 and torch.all(g == 7.0)
