"""Exhaustive GPU-vs-oracle checks of the two roundings the path performs,
over all 2**32 fp32 bit patterns, bit for bit:

* the bf16 cast (fsdp_cast_unshard_bf16) against oracle.step.bf16_rne;
* the fp8 codes (fsdp_mt_cast_fp8 with amax 448, so the scale is exactly 1
  and every code is the plain E4M3 rounding of the saturated fp32 value)
  against oracle.fp8.quantize.  NaN codes compare as NaN (IEEE 754 leaves the
  sign of a NaN result unspecified; finite and infinite inputs are exact).

The patterns are generated on the device in chunks of 2**28; the oracle runs
on the host's cores in sub-chunks.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from oracle import step as O
from rank_step_amd import binding as B

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
SUB = 1 << 24


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _patterns(c, dev):
    lo = c * CHUNK
    x = torch.arange(lo, lo + CHUNK, dtype=torch.int64, device=dev)
    return x.to(torch.int32).view(torch.float32)        # two's-complement wrap = the bit pattern


def _host_check(bits_u32, got, ref_fn, nan_free_sign):
    def one(i):
        a, b = i * SUB, (i + 1) * SUB
        f = bits_u32[a:b].view(np.float32)
        with np.errstate(all="ignore"):
            ref = ref_fn(f)
        g = got[a:b]
        if nan_free_sign:
            nan = (ref & 0x7F) == 0x7F
            bad = np.where(nan, (g & 0x7F) != 0x7F, g != ref)
        else:
            bad = g != ref
        return int(bad.sum()), (int(np.flatnonzero(bad)[0]) + a if bad.any() else -1)
    with ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(one, range(len(got) // SUB)))
    return sum(r[0] for r in res), max(r[1] for r in res)


def test_bf16_cast_all_fp32_patterns(gpu):
    out = torch.empty(CHUNK, dtype=torch.int16, device=gpu)
    base = np.arange(CHUNK, dtype=np.uint32)
    for c in range(1 << 32 >> 28):
        x = _patterns(c, gpu)
        B.fsdp_cast_unshard_bf16(out, x, CHUNK, CHUNK)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16)
        bits = base + np.uint32(c * CHUNK)
        nbad, first = _host_check(bits, got, lambda f: O.bf16_rne(f.astype(np.float64)), False)
        print(f"bf16 chunk {c:2d}: {nbad} mismatches", flush=True)
        assert nbad == 0, f"chunk {c}: first mismatch at pattern {c * CHUNK + first:#010x}"


def test_fp8_codes_all_fp32_patterns(gpu):
    # a one-shard plan whose parameter holds the patterns; m, v and the slices
    # are required by the plan but untouched by the cast
    p = torch.empty(CHUNK, dtype=torch.float32, device=gpu)
    m = torch.zeros(CHUNK, dtype=torch.float32, device=gpu)
    v = torch.zeros(CHUNK, dtype=torch.float32, device=gpu)
    sl = torch.zeros(CHUNK, dtype=torch.float32, device=gpu)
    codes = torch.empty(CHUNK, dtype=torch.uint8, device=gpu)
    amax = torch.full((1,), 448.0, dtype=torch.float32, device=gpu)
    scale = torch.zeros(1, dtype=torch.float32, device=gpu)
    plan = B.MtPlan([{"param_fp32": p, "exp_avg": m, "exp_avg_sq": v, "grad_slices": sl,
                      "slice_stride": CHUNK, "shard_numel": CHUNK, "valid": CHUNK,
                      "unshard_fp8_out": codes}], 1, "f32")
    base = np.arange(CHUNK, dtype=np.uint32)
    for c in range(1 << 32 >> 28):
        p.copy_(_patterns(c, gpu))
        plan.cast_fp8(amax, 1, scale)
        torch.cuda.synchronize()
        assert scale.item() == 1.0
        got = codes.cpu().numpy()
        bits = base + np.uint32(c * CHUNK)
        nbad, first = _host_check(bits, got, lambda f: F.quantize(f, np.float32(1.0)), True)
        print(f"fp8 chunk {c:2d}: {nbad} mismatches", flush=True)
        assert nbad == 0, f"chunk {c}: first mismatch at pattern {c * CHUNK + first:#010x}"
    plan.close()
