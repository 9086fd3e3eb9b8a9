"""Host-side checks of librank_step.so (CPU only, no device work).

* the library loads and exports every function include/*.h declares;
* fsdp_shard_layout (host C++) is bit-exact against the oracle's layout over
  an exhaustive small grid and every rank of the five workloads;
* every invalid argument is rejected with its error code before any device
  work: the cases below carry fake device addresses that are never touched.
"""

import ctypes
import glob
import itertools
import os
import re

import pytest

from oracle import layout as OL
from rank_step_amd import binding as B
from rank_step_amd.workloads import HPARAMS, WORKLOADS, shapes_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fsdp_\w+)\s*\(", text, flags=re.M))
    return names


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 9
    L = ctypes.CDLL(B.lib_path())
    missing = [n for n in sorted(names) if not hasattr(L, n)]
    assert not missing, missing
    assert set(B.EXPORTS) == names


# ---------------------------------------------------------------- layout parity

MODES = {"flat": OL.FLAT, "shard0": OL.SHARD0, "owner": OL.OWNER}


def _cmp(mode, N, shapes, has_master):
    for r in range(N):
        got_v, got_s = B.fsdp_shard_layout(mode, N, r, shapes, has_master)
        ref_v, ref_s = OL.layout(MODES[mode], N, r, shapes, has_master)
        assert got_v == [v.__dict__ for v in ref_v], (mode, N, r)
        assert got_s == ref_s.__dict__, (mode, N, r)


def test_layout_flat_exhaustive_small():
    for N in range(1, 10):
        for numels in itertools.product([0, 1, 2, 5, 7, 16], repeat=3):
            _cmp("flat", N, [(n, max(n, 1), "f32") for n in numels], False)
        for P in range(0, 65):
            _cmp("flat", N, [(P, max(P, 1), "bf16")], True)


def test_layout_shard0_exhaustive_small():
    for N in range(1, 10):
        shapes = []
        for d0 in range(0, 21):
            for row in (1, 2, 3):
                shapes.append((d0 * row, max(d0, 1), "f32" if row % 2 else "bf16"))
        _cmp("shard0", N, shapes, True)
        _cmp("shard0", N, shapes, False)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_layout_workloads_every_rank(cfg):
    w = WORKLOADS[cfg]
    _cmp(w.mode, w.world_size, shapes_of(w), w.has_master)


def test_layout_errors_leave_outputs_untouched():
    n = 2
    arr = (B.TensorShape * n)(B.TensorShape(4, 2, 0, 0), B.TensorShape(6, 4, 0, 0))
    views = (B.ShardView * n)()
    for v in views:
        v.shard_numel = 777
    summ = B.LayoutSummary()
    summ.logical_numel = 555
    rc = B.lib().fsdp_shard_layout(1, 2, 0, arr, n, 0, views, ctypes.byref(summ))
    assert rc == -1                                  # 6 is not a multiple of 4
    assert all(v.shard_numel == 777 for v in views) and summ.logical_numel == 555
    assert b"multiple" in B.lib().fsdp_last_error()


@pytest.mark.parametrize("args,code", [
    (("bogus", 2, 0, [(4, 4, "f32")], False), "ARG"),
    ((7, 2, 0, [(4, 4, "f32")], False), "ARG"),
    (("flat", 0, 0, [(4, 4, "f32")], False), "ARG"),
    (("flat", 2, 2, [(4, 4, "f32")], False), "ARG"),
    (("flat", 2, -1, [(4, 4, "f32")], False), "ARG"),
    (("flat", 2, 0, [(-4, 4, "f32")], False), "ARG"),
    (("shard0", 2, 0, [(6, 4, "f32")], False), "ARG"),
    (("shard0", 2, 0, [(6, 0, "f32")], False), "ARG"),
    (("flat", 2, 0, [(4, 4, 5)], False), "DTYPE"),
    (("flat", 2, 0, [(4, 4, "f32"), (4, 4, "bf16")], False), "DTYPE"),
    (("flat", 2, 0, [(2 ** 62, 1, "f32"), (2 ** 62, 1, "f32")], False), "ARG"),
])
def test_layout_invalid(args, code):
    mode = args[0]
    if mode == "bogus":
        args = (9,) + args[1:]
    with pytest.raises(B.FsdpError) as e:
        B.fsdp_shard_layout(*args)
    assert e.value.name == "FSDP_E_" + code


def test_layout_reserved_must_be_zero():
    arr = (B.TensorShape * 1)(B.TensorShape(4, 4, 0, 1))
    views = (B.ShardView * 1)()
    assert B.lib().fsdp_shard_layout(0, 1, 0, arr, 1, 0, views, None) == -1


def test_layout_empty_unit():
    v, s = B.fsdp_shard_layout("flat", 4, 3, [], False)
    assert v == [] and s["shard_numel"] == 0 and s["physical_numel"] == 0


# ---------------------------------------------------------------- argument checks of device calls
# Fake device addresses: 16-byte aligned, far apart, never dereferenced
# because every case fails validation on the host.
A, Bp, C, D, E, F = (0x100000000 * k for k in range(1, 7))
HP = dict(HPARAMS)


def _err(fn, *a, **k):
    with pytest.raises(B.FsdpError) as e:
        fn(*a, **k)
    return e.value.name[len("FSDP_E_"):]


def test_reduce_argument_checks():
    f = B.fsdp_reduce_grad_shard
    assert _err(f, A, Bp, "f32", 100, 0, 100, 100, stream=0) == "ARG"       # N = 0
    assert _err(f, A, Bp, "f32", 100, 1025, 100, 100, stream=0) == "ARG"    # N too large
    assert _err(f, A, Bp, "f32", 99, 4, 100, 100, stream=0) == "ARG"        # stride < S
    assert _err(f, A, Bp, "f32", 100, 4, 100, 101, stream=0) == "ARG"       # valid > S
    assert _err(f, A, Bp, "f32", 100, 4, -1, 0, stream=0) == "ARG"          # negative S
    assert _err(f, None, Bp, "f32", 100, 4, 100, 100, stream=0) == "ARG"    # null out
    assert _err(f, A, None, "f32", 100, 4, 100, 100, stream=0) == "ARG"     # null slices
    assert _err(f, A, Bp, 3, 100, 4, 100, 100, stream=0) == "DTYPE"
    assert _err(f, A + 2, Bp, "f32", 100, 4, 100, 100, stream=0) == "ALIGN"
    assert _err(f, A, Bp + 1, "bf16", 100, 4, 100, 100, stream=0) == "ALIGN"
    # output inside slice 2 of 4
    assert _err(f, Bp + 2 * 400 + 16, Bp, "f32", 100, 4, 100, 100, stream=0) == "ALIAS"
    assert _err(f, A, Bp, "f32", 2 ** 62, 8, 100, 100, stream=0) == "ARG"    # extent overflow
    B.fsdp_reduce_grad_shard(None, None, "f32", 0, 4, 0, 0, stream=0)       # S = 0: no-op


def test_adamw_argument_checks():
    f = B.fsdp_adamw_shard_step
    ok = (A, Bp, C, D, 100, 100)
    assert _err(f, *ok, dict(HP, beta1=1.0), 1, stream=0) == "ARG"
    assert _err(f, *ok, dict(HP, beta2=-0.1), 1, stream=0) == "ARG"
    assert _err(f, *ok, dict(HP, lr=float("nan")), 1, stream=0) == "ARG"
    assert _err(f, *ok, dict(HP, eps=-1e-8), 1, stream=0) == "ARG"
    assert _err(f, *ok, dict(HP, weight_decay=-1.0), 1, stream=0) == "ARG"
    assert _err(f, *ok, HP, 0, stream=0) == "ARG"                            # step < 1
    assert _err(f, None, Bp, C, D, 100, 100, HP, 1, stream=0) == "ARG"
    assert _err(f, A, Bp, C, None, 100, 100, HP, 1, stream=0) == "ARG"
    assert _err(f, A + 1, Bp, C, D, 100, 100, HP, 1, stream=0) == "ALIGN"
    assert _err(f, A, A + 200, C, D, 100, 100, HP, 1, stream=0) == "ALIAS"  # m overlaps p
    assert _err(f, A, Bp, C, C + 16, 100, 100, HP, 1, stream=0) == "ALIAS"  # grad inside v
    B.fsdp_adamw_shard_step(None, None, None, None, 0, 0, HP, 1, stream=0)


def test_cast_argument_checks():
    f = B.fsdp_cast_unshard_bf16
    assert _err(f, None, A, 100, 100, stream=0) == "ARG"
    assert _err(f, Bp, None, 100, 100, stream=0) == "ARG"
    assert _err(f, Bp + 1, A, 100, 100, stream=0) == "ALIGN"
    assert _err(f, A + 100, A, 100, 100, stream=0) == "ALIAS"
    assert _err(f, Bp, A, 100, 101, stream=0) == "ARG"


def _t(p, m, v, s, S=1024, valid=1024, out=None, gout=None, stride=None):
    return {"param_fp32": p, "exp_avg": m, "exp_avg_sq": v, "grad_slices": s,
            "slice_stride": S if stride is None else stride, "unshard_bf16_out": out,
            "grad_shard_out": gout, "shard_numel": S, "valid": valid}


def test_mt_plan_argument_checks():
    f = B.fsdp_mt_plan_create
    base = [_t(A, A + 8192, A + 16384, Bp, out=C), _t(D, D + 8192, D + 16384, Bp + 8192, out=C + 4096)]
    bad_alias = [base[0], _t(D, D + 8192, A + 8192 + 100, Bp + 8192)]    # shard 1 v inside shard 0 m
    assert _err(f, bad_alias, 2, "f32", stream=0) == "ALIAS"
    bad_out = [base[0], _t(D, D + 8192, D + 16384, Bp + 8192, out=C + 1000)]   # bf16 outputs overlap
    assert _err(f, bad_out, 2, "f32", stream=0) == "ALIAS"
    slice_in_param = [_t(A, A + 8192, A + 16384, A + 4, stride=1024)]
    assert _err(f, slice_in_param, 1, "f32", stream=0) == "ALIAS"
    assert _err(f, [_t(None, A, Bp, C)], 1, "f32", stream=0) == "ARG"
    assert _err(f, [_t(A, Bp, C, D, S=10, valid=11)], 1, "f32", stream=0) == "ARG"
    assert _err(f, [_t(A + 2, Bp, C, D)], 1, "f32", stream=0) == "ALIGN"
    assert _err(f, [_t(A, Bp, C, D, stride=100)], 2, "f32", stream=0) == "ARG"
    assert _err(f, base, 0, "f32", stream=0) == "ARG"
    assert _err(f, base, 2, 9, stream=0) == "DTYPE"
    # overlapping read-only slices are allowed: this plan fails only on its alias
    shared = [_t(A, A + 8192, A + 16384, Bp), _t(D, D + 8192, D + 16384, Bp, out=A + 100)]
    assert _err(f, shared, 1, "f32", stream=0) == "ALIAS"


def test_mt_step_and_destroy_null():
    assert B.lib().fsdp_mt_step(None, None, None) == -1
    assert B.lib().fsdp_mt_plan_destroy(None) == 0
    assert B.lib().fsdp_mt_plan_get_info(None, None) == -1


def test_clip_argument_checks():
    f = B.fsdp_clip_coef
    assert _err(f, None, None, A, 1, 1.0, stream=0) == "ARG"
    assert _err(f, Bp, None, None, 1, 1.0, stream=0) == "ARG"
    assert _err(f, Bp, None, A, 0, 1.0, stream=0) == "ARG"
    assert _err(f, Bp, None, A, 4, float("nan"), stream=0) == "ARG"
    assert _err(f, Bp, None, A, 4, -1.0, stream=0) == "ARG"
    assert _err(f, Bp + 2, None, A, 4, 1.0, stream=0) == "ALIGN"
    assert _err(f, Bp, C + 4, A, 4, 1.0, stream=0) == "ALIGN"
    assert _err(f, A + 8, None, A, 4, 1.0, stream=0) == "ALIAS"     # coef inside the sums
    assert _err(f, Bp, Bp, A, 4, 1.0, stream=0) == "ALIAS"          # both outputs at one address
    assert B.lib().fsdp_mt_reduce_sqnorm(None, A, None) == -1
    assert B.lib().fsdp_mt_step_clipped(None, None, A, None) == -1


def test_accumulate_argument_checks():
    f = B.fsdp_grad_accumulate
    assert _err(f, None, A, "f32", 100, 1, stream=0) == "ARG"
    assert _err(f, A, None, "bf16", 100, 1, stream=0) == "ARG"
    assert _err(f, A, Bp, 7, 100, 1, stream=0) == "DTYPE"
    assert _err(f, A, Bp, "f32", -1, 1, stream=0) == "ARG"
    assert _err(f, A + 2, Bp, "f32", 100, 1, stream=0) == "ALIGN"
    assert _err(f, A, Bp + 1, "bf16", 100, 1, stream=0) == "ALIGN"
    assert _err(f, A, A + 200, "f32", 100, 1, stream=0) == "ALIAS"
    assert B.lib().fsdp_grad_accumulate(A, Bp, 0, 100, 2, None) == -1    # accumulate not 0/1
    B.fsdp_grad_accumulate(None, None, "f32", 0, 1, stream=0)              # empty: no-op
    assert B.lib().fsdp_mt_reduce_accumulate(None, 0, None, None) == -1
    assert B.lib().fsdp_mt_step_amax(None, None, A, None) == -1
    assert B.lib().fsdp_mt_cast_fp8(None, A, 1, None, None) == -1
    assert B.lib().fsdp_mt_step_fp8(None, None, A, Bp, None) == -1


def test_layout_owner_matches_oracle():
    import random
    rnd = random.Random(5)
    for _ in range(100):
        N = rnd.randint(1, 9)
        shapes = [(rnd.choice([0, 1, 7, 64, 4096, 5000]) * rnd.randint(1, 3), 1,
                   rnd.choice(["f32", "bf16"])) for _ in range(rnd.randint(0, 10))]
        shapes = [(n, max(n, 1), d) for n, _, d in shapes]
        _cmp("owner", N, shapes, rnd.random() < 0.5)
    for cfg in (2, 4):
        w = WORKLOADS[cfg]
        _cmp("owner", w.world_size, shapes_of(w), w.has_master)


def test_capacity_error_before_any_device_work():
    # 2**44 elements need more workgroups of 256 than one launch holds: refused on the host
    big = 1 << 44
    assert _err(B.fsdp_cast_unshard_bf16, A, None, big, 0, stream=0) == "CAPACITY"
    assert _err(B.fsdp_reduce_grad_shard, A, None, "f32", big, 1, big, 0, stream=0) == "CAPACITY"


def test_plan_capacity_checked_before_its_table_is_built():
    # a shard of 2**44 elements needs 2**33 chunk entries (128 GiB of host
    # table): the plan is refused from the launch size alone, at once and
    # without building any of it (fake device addresses, never touched)
    import time
    big = 1 << 44
    t0 = time.perf_counter()
    huge = [_t(1 << 40, 2 << 46, 3 << 46, 4 << 46, S=big, valid=big, stride=big)]
    assert _err(B.fsdp_mt_plan_create, huge, 1, "f32", stream=0) == "CAPACITY"
    # the same total spread over many shards
    many = [_t((k + 1) << 42, (k + 1) << 42 | (1 << 41), (k + 65) << 42, (k + 129) << 42,
               S=1 << 33, valid=1 << 33, stride=1 << 33) for k in range(40)]
    assert _err(B.fsdp_mt_plan_create, many, 1, "f32", stream=0) == "CAPACITY"
    assert time.perf_counter() - t0 < 5.0


def test_layout_extreme_sizes_match_oracle_or_refuse():
    # sizes far beyond any device, where 32-bit or careless 64-bit arithmetic
    # would wrap: the library agrees with the oracle's exact integers ...
    big = [("flat", 1 << 30, [(7, 7, "f32")], True),
           ("shard0", 1000, [((1 << 40), (1 << 20), "bf16")], True),
           ("flat", 3, [((1 << 40) + 1, 1, "f32"), ((1 << 41) + 1, 3, "f32")], False),
           ("owner", 7, [((1 << 40) + k, 1, "bf16") for k in range(9)], True)]
    for mode, N, shapes, master in big:
        for r in (0, 1, N // 2, N - 1):
            got_v, got_s = B.fsdp_shard_layout(mode, N, r, shapes, master)
            ref_v, ref_s = OL.layout(MODES[mode], N, r, shapes, master)
            assert got_v == [v.__dict__ for v in ref_v], (mode, N, r)
            assert got_s == ref_s.__dict__, (mode, N, r)
    # ... or refuses when a count or byte total would not fit in int64
    for mode, N, shapes in (("flat", 3, [((1 << 62), 1, "f32")] * 2),
                            ("owner", 4, [((1 << 61), 1, "f32")] * 3),
                            ("flat", 8, [((1 << 61), 1, "f32")] * 5)):
        assert _err(B.fsdp_shard_layout, mode, N, 0, shapes, True) == "ARG"


def test_last_error_is_per_thread():
    # four threads fail concurrently with different ranks; each must read back
    # the message of its own last failing call (ctypes drops the GIL in calls)
    import threading
    L = B.lib()
    shape = (B.TensorShape * 1)(B.TensorShape(4, 4, 0, 0))
    views = (B.ShardView * 1)()
    summ = B.LayoutSummary()
    bad = []

    def worker(k):
        rank = 100 + k
        for _ in range(2000):
            rc = L.fsdp_shard_layout(0, 2, rank, shape, 1, 0, views, ctypes.byref(summ))
            msg = L.fsdp_last_error().decode()
            if rc != -1 or f"rank {rank} " not in msg:
                bad.append((k, rc, msg))
                return

    ts = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad[:3]


def test_mt_plan_slice_table_checks():
    # a shard whose N slices sit in separate buffers (a table of pointers);
    # fake device addresses, refused before any device work
    f = B.fsdp_mt_plan_create

    def tab(ptrs, valid=1024):
        t = _t(A, A + 8192, A + 16384, None, valid=valid)
        t.pop("grad_slices")
        t["grad_slice_ptrs"] = ptrs
        return t

    assert _err(f, [tab([Bp, None, C])], 3, "f32", stream=0) == "ARG"          # a null entry
    assert _err(f, [tab([Bp, C + 2, D])], 3, "f32", stream=0) == "ALIGN"       # not 4-byte aligned
    assert _err(f, [tab([Bp, C + 1, D])], 3, "bf16", stream=0) == "ALIGN"      # not 2-byte aligned
    assert _err(f, [tab([Bp, A + 400, D])], 3, "f32", stream=0) == "ALIAS"     # inside param
    # another shard's written buffer overlapping a table entry
    other = _t(E, E + 8192, E + 16384, F)
    assert _err(f, [tab([Bp, C, E + 100]), other], 3, "f32", stream=0) == "ALIAS"
