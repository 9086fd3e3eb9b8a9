"""fsdp_rank_buffer_layout (host only): where one rank's step buffers go in one
allocation.  Checked here: every region starts on its 2 MiB boundary, in the
stated order, without overlap and within total_bytes; the slice rows are
shard_numel rounded up to 64 elements plus 256 apart (shard_numel for one
slice), so bf16 rows start on 128-byte lines; absent buffers are -1; the
argument errors; and the workloads' placements, which the tests and the
benchmark allocate through it."""

import ctypes
import random

import pytest

from rank_step_amd import binding as B
from rank_step_amd.workloads import WORKLOADS, shapes_of

RA = 2 << 20
ORDER = [("param_offset", 4), ("exp_avg_offset", 4), ("exp_avg_sq_offset", 4), ("slices_offset", None),
         ("bf16_offset", 2), ("grad_out_offset", 4), ("fp8_offset", 1)]


def _sizes(S, N, sdt, slots, go, f8, stride):
    es = 2 if sdt == "bf16" else 4
    return {"param_offset": 4 * S, "exp_avg_offset": 4 * S, "exp_avg_sq_offset": 4 * S,
            "slices_offset": es * N * stride, "bf16_offset": 2 * S * slots if slots else None,
            "grad_out_offset": 4 * S if go else None, "fp8_offset": S if f8 else None}


def _check(S, N, sdt, slots, go, f8):
    lay = B.fsdp_rank_buffer_layout(S, N, sdt, slots, go, f8)
    assert lay["region_align"] == RA
    stride = lay["slice_stride"]
    if N == 1:
        assert stride == S
    else:
        assert stride == -(-S // 64) * 64 + 256
        assert (stride * (2 if sdt == "bf16" else 4)) % 128 == 0
    sizes = _sizes(S, N, sdt, slots, go, f8, stride)
    end = 0
    for name, _ in ORDER:
        off = lay[name]
        if sizes[name] is None:
            assert off == -1, name
            continue
        assert off % RA == 0 and off >= end, (name, off, end)
        assert off < end + RA, (name, off, end)        # the first boundary at or after the last end
        end = off + sizes[name]
    assert lay["total_bytes"] == end
    return lay


def test_regions_are_aligned_ordered_and_disjoint():
    rng = random.Random(11)
    for _ in range(3000):
        S = rng.choice([0, 1, 3, 63, 64, 65, 255, 256, 2047, 2048, rng.randrange(1, 1 << 31)])
        N = rng.choice([1, 2, 3, 8, 32, 1024])
        _check(S, N, rng.choice(["f32", "bf16"]), rng.choice([0, 1, 8, 64]), rng.choice([0, 1]),
               rng.choice([0, 1]))


def test_workload_placements():
    """The harness (rank_step_amd/state.py) allocates every workload's rank
    through this call: the 7B shard's slice rows are 842,301,952 + 256
    elements apart, and each region starts on a 2 MiB boundary."""
    for cfg, w in WORKLOADS.items():
        _, summ = B.fsdp_shard_layout(w.mode, w.world_size, 0, shapes_of(w), w.has_master)
        S = summ["shard_numel"]
        lay = _check(S, w.n_slices, w.slice_dtype, 1 if w.bf16_out else 0, 0, 0)
        if w.n_slices > 1:
            assert S % 64 == 0 and lay["slice_stride"] == S + 256, w.name
    lay = B.fsdp_rank_buffer_layout(842301952, 8, "bf16", 1)
    assert lay["slice_stride"] == 842302208
    assert lay["exp_avg_offset"] == -(-842301952 * 4 // RA) * RA


def test_refusals():
    for args, code in [((-1, 2, "f32"), "FSDP_E_ARG"), ((10, 0, "f32"), "FSDP_E_ARG"),
                       ((10, 1025, "f32"), "FSDP_E_ARG"), ((10, 2, "f32", -1), "FSDP_E_ARG"),
                       ((1 << 62, 1024, "bf16"), "FSDP_E_ARG")]:
        with pytest.raises(B.FsdpError, match=code):
            B.fsdp_rank_buffer_layout(*args)
    # flags other than 0 and 1, an unknown dtype code and a null output,
    # through the raw call (the binding passes flags as 0 or 1)
    out = B.RankBuffers()
    assert B.lib().fsdp_rank_buffer_layout(10, 2, 0, 1, 2, 0, ctypes.byref(out)) == -1
    assert B.lib().fsdp_rank_buffer_layout(10, 2, 0, 1, 0, -1, ctypes.byref(out)) == -1
    assert B.lib().fsdp_rank_buffer_layout(10, 2, 7, 1, 0, 0, ctypes.byref(out)) == -2
    assert B.lib().fsdp_rank_buffer_layout(10, 2, 0, 1, 0, 0, None) == -1
