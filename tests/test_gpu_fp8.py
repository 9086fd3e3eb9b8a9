"""GPU parity of the fp8 all-gather copy with per-tensor scales.

Integer decisions (the per-tensor amax as fp32 bits, the fp32 scale and every
fp8 code) are compared bit for bit with the oracle applied to the GPU's own
updated fp32 parameters, which are themselves checked against the oracle's
step within the fp32 tolerance.  Covered: every rank of the tiny MLP with the
cross-rank amax combine, a Llama block (9 tensors), ragged / misaligned /
padded / empty shards, NaN propagation, bit-identity of the amax step with the
plain fused step, and the 7B rank shard (291 tensors) at full size.
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from oracle import step as O
from rank_step_amd import binding as B
from rank_step_amd.state import RankState
from rank_step_amd.workloads import HPARAMS, WORKLOADS
from tests import parity as PR

pytestmark = pytest.mark.gpu


def _codes(t):
    return t.cpu().numpy().astype(np.uint8)


def _check_codes(name, p_f32, codes, scale):
    """Codes bit-exact to the oracle's; for NaN codes only the NaN pattern is
    compared, since IEEE 754 leaves the sign of a NaN result unspecified."""
    ref = F.quantize(p_f32, scale)
    nan = (ref & 0x7F) == 0x7F
    bad = np.where(nan, (codes & 0x7F) != 0x7F, ref != codes)
    assert not bad.any(), f"{name}: {bad.sum()} codes differ, first at {np.flatnonzero(bad)[:5]}"


def test_tiny_mlp_every_rank_cross_rank_amax(gpu):
    w = WORKLOADS[1]
    N = w.world_size
    states = [RankState(w, r, gpu, bf16_out=True, fp8_out=True) for r in range(N)]
    for st in states:
        st.make_plan()
    amax = torch.zeros(N, 1, dtype=torch.float32, device=gpu)
    scale = torch.zeros(N, 1, dtype=torch.float32, device=gpu)
    for t in range(1, w.steps + 1):
        snaps = []
        for r, st in enumerate(states):
            st.load_grads(t)
            snaps.append((PR.f64(st.master), PR.f64(st.exp_avg), PR.f64(st.exp_avg_sq),
                          PR.widen_slices(st.slices, w.slice_dtype)))
            st.plan.step_amax(w.hparams, t, amax[r])
        for r, st in enumerate(states):
            st.plan.cast_fp8(amax, N, scale[r])
        torch.cuda.synchronize()
        ps = [st.master.cpu().numpy() for st in states]
        for r, (st, snap) in enumerate(zip(states, snaps)):
            ref = O.rank_step(*snap[:3], snap[3], st.total, t, w.hparams)
            fl = PR.floors(*snap[:3], snap[3], ref, w.hparams, t)
            PR.assert_close(f"fp8 rank {r} t={t} p", ps[r], ref["p"], fl["p"])
            assert np.float32(amax[r, 0].item()) == np.float32(F.amax(ps[r]))
        g_amax = max(F.amax(p) for p in ps)
        sc = F.scale_of(g_amax)
        for r, st in enumerate(states):
            assert np.float32(scale[r, 0].item()) == sc
            _check_codes(f"fp8 rank {r} t={t}", ps[r], _codes(st.fp8), sc)
    for st in states:
        st.close()


def test_amax_step_is_the_fused_step_bitwise_and_block_codes(gpu):
    w = WORKLOADS[3]
    a = RankState(w, 0, gpu, bf16_out=True, fp8_out=True)
    b = RankState(w, 0, gpu, bf16_out=True, fp8_out=True)
    a.make_plan()
    b.make_plan()
    n = len(a.segments)
    amax = torch.zeros(n, dtype=torch.float32, device=gpu)
    scale = torch.zeros(n, dtype=torch.float32, device=gpu)
    for t in (1, 2):
        a.load_grads(t)
        b.load_grads(t)
        a.step(t)
        b.plan.step_amax(w.hparams, t, amax)
        b.plan.cast_fp8(amax, 1, scale)
        torch.cuda.synchronize()
        for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(a.ag.view(torch.int16), b.ag.view(torch.int16))
        p = b.master.cpu().numpy()
        codes = _codes(b.fp8)
        am = amax.cpu().numpy()
        sc = scale.cpu().numpy()
        for i, (off, length, held, _) in enumerate(b.segments):
            seg = p[off:off + held]
            assert am[i] == np.float32(F.amax(seg)), i
            assert sc[i] == F.scale_of(am[i]), i
            _check_codes(f"block tensor {i} t={t}", seg, codes[off:off + held], sc[i])
    a.close()
    b.close()


SPECS = [(0, 0, 0), (1, 1, 0), (7, 0, 0), (8, 8, 0), (2048 * 5 + 1237, 2048 * 5 + 1230, 0),
         (9001, 8999, 1), (4096, 3, 0), (70001, 70001, 0),
         # one and a bit of the code pass's 1024-element spans; 4-byte aligned codes
         (1024, 1024, 0), (1025, 1021, 0), (2048 * 3 + 1100, 2048 * 3 + 1100, 4)]


def test_ragged_shards_and_nan(gpu):
    N, sdt = 3, "bf16"
    g = torch.Generator(device=gpu)
    g.manual_seed(5)
    shards = []
    for i, (S, valid, off) in enumerate(SPECS):
        base = lambda n, dt: torch.zeros(n + off, dtype=dt, device=gpu)[off:]
        p = base(S, torch.float32)
        p[:valid] = torch.randn(valid, generator=g, device=gpu) * 0.02
        m, v = base(S, torch.float32), base(S, torch.float32)
        sl = torch.zeros(N * S + off, dtype=torch.bfloat16, device=gpu)[off:]
        sl[:] = (torch.randn(N * S, generator=g, device=gpu) * 1e-2).to(torch.bfloat16)
        f8 = torch.full((S + off,), 0xAB, dtype=torch.uint8, device=gpu)[off:]
        shards.append(dict(p=p, m=m, v=v, sl=sl, f8=f8, S=S, valid=valid))
    # a NaN gradient in shard 4 makes that tensor's amax, scale and codes NaN
    shards[4]["sl"][17] = float("nan")
    plan = B.MtPlan([{"param_fp32": s["p"], "exp_avg": s["m"], "exp_avg_sq": s["v"],
                      "grad_slices": s["sl"], "slice_stride": s["S"], "shard_numel": s["S"],
                      "valid": s["valid"], "unshard_fp8_out": s["f8"]} for s in shards], N, sdt)
    n = len(shards)
    amax = torch.full((n,), -1.0, dtype=torch.float32, device=gpu)
    scale = torch.zeros(n, dtype=torch.float32, device=gpu)
    plan.step_amax(HPARAMS, 1, amax)
    plan.cast_fp8(amax, 1, scale)
    torch.cuda.synchronize()
    am = amax.cpu().numpy()
    sc = scale.cpu().numpy()
    for i, s in enumerate(shards):
        p = s["p"].cpu().numpy()
        codes = _codes(s["f8"])
        ref_am = F.amax(p[:s["valid"]])
        if np.isnan(ref_am):
            assert np.isnan(am[i]) and np.isnan(sc[i])
        else:
            assert am[i] == np.float32(ref_am), i
        if s["S"] == 0:
            continue
        scale_i = F.scale_of(am[i])
        assert (np.isnan(sc[i]) and np.isnan(scale_i)) or sc[i] == scale_i
        _check_codes(f"ragged {i}", p[:s["valid"]], codes[:s["valid"]], scale_i)
        assert np.all(codes[s["valid"]:] == 0), f"ragged {i}: pad codes not 0"
    assert np.all((_codes(shards[4]["f8"])[:shards[4]["valid"]] & 0x7F) == 0x7F)
    plan.close()


def test_llama7b_full_size(gpu):
    w = WORKLOADS[4]
    st = RankState(w, 0, gpu, bf16_out=False, fp8_out=True)
    st.make_plan()
    n = len(st.segments)
    amax = torch.zeros(n, dtype=torch.float32, device=gpu)
    scale = torch.zeros(n, dtype=torch.float32, device=gpu)
    st.load_grads(1)
    st.plan.step_amax(w.hparams, 1, amax)
    st.plan.cast_fp8(amax, 1, scale)
    torch.cuda.synchronize()
    am = amax.cpu().numpy()
    sc = scale.cpu().numpy()
    for i, (off, length, held, _) in enumerate(st.segments):
        ref = float(st.master[off:off + held].abs().max().item())     # torch's own amax
        assert am[i] == np.float32(ref), i
        assert sc[i] == F.scale_of(am[i]), i
    rng = np.random.default_rng(7)
    idx = np.unique(rng.integers(0, st.total, 1 << 20))
    idx_t = torch.from_numpy(idx).to(gpu)
    seg_of = np.searchsorted(np.array([s[0] for s in st.segments]), idx, side="right") - 1
    p = st.master[idx_t].cpu().numpy()
    codes = _codes(st.fp8[idx_t])
    ref = np.array([F.quantize(p[k:k + 1], sc[seg_of[k]])[0] for k in range(0, len(idx), 997)])
    assert np.array_equal(codes[::997], ref)
    # vectorised over all sampled elements, grouped by tensor
    for i in np.unique(seg_of):
        sel = seg_of == i
        _check_codes(f"7b tensor {i}", p[sel], codes[sel], sc[i])
    st.close()
    del st
    torch.cuda.empty_cache()


def _ragged_set(gpu, seed, N=3, sdt="bf16"):
    """The ragged/misaligned shards of SPECS, each with an fp8 output and garbage codes."""
    g = torch.Generator(device=gpu)
    g.manual_seed(seed)
    shards = []
    for S, valid, off in SPECS:
        base = lambda n, dt: torch.zeros(n + off, dtype=dt, device=gpu)[off:]
        p = base(S, torch.float32)
        p[:valid] = torch.randn(valid, generator=g, device=gpu) * 0.02
        m, v = base(S, torch.float32), base(S, torch.float32)
        sl = torch.zeros(N * S + off, dtype=torch.bfloat16, device=gpu)[off:]
        sl[:] = (torch.randn(N * S, generator=g, device=gpu) * 1e-2).to(torch.bfloat16)
        f8 = torch.full((S + off,), 0xAB, dtype=torch.uint8, device=gpu)[off:]
        shards.append(dict(p=p, m=m, v=v, sl=sl, f8=f8, S=S, valid=valid))
    plan = B.MtPlan([{"param_fp32": s["p"], "exp_avg": s["m"], "exp_avg_sq": s["v"],
                      "grad_slices": s["sl"], "slice_stride": s["S"], "shard_numel": s["S"],
                      "valid": s["valid"], "unshard_fp8_out": s["f8"]} for s in shards], N, sdt)
    return shards, plan


def test_step_fp8_with_given_scales(gpu):
    """fsdp_mt_step_fp8: fp32 outputs bit-identical to fsdp_mt_step_amax's (the
    plain step), the same amax, and codes equal to the oracle's quantisation of
    the GPU's own p' with the given scales (tiny, huge and ordinary ones)."""
    a, plan_a = _ragged_set(gpu, 31)
    b, plan_b = _ragged_set(gpu, 31)
    n = len(a)
    scales = np.array([448.0 / 0.05, 1e-30, 1e30, 448.0 / 0.02, 3.0e4, 1.0, 448.0 / 0.08, 12345.678,
                       0.5, 2.0 ** -10, 7.0e5][:n], dtype=np.float32)
    scale_in = torch.from_numpy(scales).to(gpu)
    amax_a = torch.full((n,), -1.0, dtype=torch.float32, device=gpu)
    amax_b = torch.full((n,), -1.0, dtype=torch.float32, device=gpu)
    for t in (1, 2):
        plan_a.step_fp8(HPARAMS, t, scale_in, amax_a)
        plan_b.step_amax(HPARAMS, t, amax_b)
        torch.cuda.synchronize()
        assert torch.equal(amax_a.view(torch.int32), amax_b.view(torch.int32)), t
        for i, (x, y) in enumerate(zip(a, b)):
            for k in ("p", "m", "v"):
                assert torch.equal(x[k].view(torch.int32), y[k].view(torch.int32)), (i, k, t)
            if x["S"] == 0:
                continue
            p = x["p"].cpu().numpy()
            codes = _codes(x["f8"])
            _check_codes(f"step_fp8 shard {i} t={t}", p[:x["valid"]], codes[:x["valid"]], scales[i])
            assert np.all(codes[x["valid"]:] == 0), f"step_fp8 shard {i}: pad codes not 0"
    plan_a.close()
    plan_b.close()


def test_delayed_scaling_two_steps(gpu):
    """Step 1 scales dynamically (step with amax, then the code pass); step 2
    takes step 1's scales in the one-pass fp8 step.  Step 2's codes are the
    oracle's quantisation of its own p' with step 1's scales, and its amax is
    the new |p'| maximum."""
    w = WORKLOADS[3]
    st = RankState(w, 0, gpu, bf16_out=True, fp8_out=True)
    st.make_plan(with_grad_out=False)
    n = len(st.segments)
    amax = torch.zeros(n, dtype=torch.float32, device=gpu)
    scale1 = torch.zeros(n, dtype=torch.float32, device=gpu)
    st.load_grads(1)
    st.plan.step_amax(w.hparams, 1, amax)
    st.plan.cast_fp8(amax, 1, scale1)
    st.load_grads(2)
    st.plan.step_fp8(w.hparams, 2, scale1, amax)
    torch.cuda.synchronize()
    sc = scale1.cpu().numpy()
    am = amax.cpu().numpy()
    for i, (off, length, held, _) in enumerate(st.segments):
        p = st.master[off:off + held].cpu().numpy()
        assert am[i] == np.float32(F.amax(p)), i
        _check_codes(f"delayed shard {i}", p, _codes(st.fp8[off:off + held]), sc[i])
        bf = PR.bf16_bits(st.ag_slot[off:off + held])
        assert np.array_equal(bf, O.bf16_rne(p.astype(np.float64))), i
    st.close()


@pytest.mark.parametrize("f8_off", [1, 2, 3])
def test_fp8_codes_at_any_byte_alignment(gpu, f8_off):
    """fp8 copies 1-3 bytes past a 4-byte boundary, the fp32 state aligned:
    the code pass and the one-pass fp8 step store them in narrower pieces.
    Codes equal the oracle's quantisation of the GPU's own p', the padding
    codes are 0 and the bytes around every copy are untouched."""
    N, sdt = 3, "bf16"
    sizes = [(2048 * 3 + 1100, 2048 * 3 + 1093), (1025, 1021), (37, 37)]
    g = torch.Generator(device=gpu)
    g.manual_seed(90 + f8_off)
    shards = []
    for S, valid in sizes:
        p = torch.zeros(S, dtype=torch.float32, device=gpu)
        p[:valid] = torch.randn(valid, generator=g, device=gpu) * 0.02
        m, v = torch.zeros_like(p), torch.zeros_like(p)
        sl = (torch.randn(N * S, generator=g, device=gpu) * 1e-2).to(torch.bfloat16)
        raw = torch.full((S + 16,), 0xAB, dtype=torch.uint8, device=gpu)
        shards.append(dict(p=p, m=m, v=v, sl=sl, raw=raw, f8=raw[8 + f8_off:8 + f8_off + S],
                           S=S, valid=valid))
    plan = B.MtPlan([{"param_fp32": s["p"], "exp_avg": s["m"], "exp_avg_sq": s["v"],
                      "grad_slices": s["sl"], "slice_stride": s["S"], "shard_numel": s["S"],
                      "valid": s["valid"], "unshard_fp8_out": s["f8"]} for s in shards], N, sdt)
    n = len(shards)

    def check(name, scales):
        for i, s in enumerate(shards):
            p = s["p"].cpu().numpy()
            codes = _codes(s["f8"])
            _check_codes(f"{name} shard {i}", p[:s["valid"]], codes[:s["valid"]], scales[i])
            assert np.all(codes[s["valid"]:] == 0), f"{name} shard {i}: pad codes not 0"
            raw = _codes(s["raw"])
            lo, hi = 8 + f8_off, 8 + f8_off + s["S"]
            assert np.all(raw[:lo] == 0xAB) and np.all(raw[hi:] == 0xAB), f"{name} shard {i}: guard bytes"

    # dynamic scaling: the step with amax, then the code pass
    amax = torch.full((n,), -1.0, dtype=torch.float32, device=gpu)
    scale = torch.zeros(n, dtype=torch.float32, device=gpu)
    plan.step_amax(HPARAMS, 1, amax)
    plan.cast_fp8(amax, 1, scale)
    torch.cuda.synchronize()
    am = amax.cpu().numpy()
    for i, s in enumerate(shards):
        assert am[i] == np.float32(F.amax(s["p"].cpu().numpy()[:s["valid"]])), i
    check("code pass", [F.scale_of(a) for a in am])
    # the one-pass step with given scales
    scales = np.array([448.0 / 0.05, 3.0e4, 0.5], dtype=np.float32)
    plan.step_fp8(HPARAMS, 2, torch.from_numpy(scales).to(gpu), amax)
    torch.cuda.synchronize()
    check("one-pass step", scales)
    plan.close()


def _monotone_e4m3(c):
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def test_codes_against_the_double_trajectory(gpu):
    """The codes against the oracle taken wholly in double precision: the
    updated parameter from the oracle's step (per-step resync), each tensor's
    amax and scale 448 / max(amax, 1e-12) in double, and the code
    RNE_e4m3(clamp(p' * scale)) in double.  The GPU decides the same code in
    fp32 from its own p' and scale, so the two may differ by one code step
    where p' * scale lies within its fp32 allowance of a rounding boundary:
    wherever that allowance is below half an fp8 step, a code must be within
    one step of the double one.  Reported: the codes that differ at all."""
    w = WORKLOADS[3]
    st = RankState(w, 0, gpu, bf16_out=True, fp8_out=True)
    st.make_plan()
    n = len(st.segments)
    amax = torch.zeros(n, dtype=torch.float32, device=gpu)
    scale = torch.zeros(n, dtype=torch.float32, device=gpu)
    differ = 0
    judged_total = 0
    for t in (1, 2, 3):
        st.load_grads(t)
        snap = (PR.f64(st.master), PR.f64(st.exp_avg), PR.f64(st.exp_avg_sq),
                PR.widen_slices(st.slices, w.slice_dtype))
        st.plan.step_amax(w.hparams, t, amax)
        st.plan.cast_fp8(amax, 1, scale)
        torch.cuda.synchronize()
        codes = _codes(st.fp8)
        am = amax.cpu().numpy()
        for i, (off, length, held, _) in enumerate(st.segments):
            a, b = off, off + held
            p0, m0, v0, sl = (x[..., a:b] for x in snap)
            ref = O.rank_step(p0, m0, v0, sl, held, t, w.hparams)
            fl = PR.floors(p0, m0, v0, sl, ref, w.hparams, t)
            amax_ref = float(np.max(np.abs(ref["p"])))
            assert abs(float(am[i]) - amax_ref) <= PR.TOL * amax_ref, (i, float(am[i]), amax_ref)
            sc = F.E4M3_MAX / max(amax_ref, F.AMAX_FLOOR)
            y = np.clip(ref["p"] * sc, -F.E4M3_MAX, F.E4M3_MAX)
            q_ref = F.e4m3_rne(y)
            got = codes[a:b]
            ay = np.abs(y)
            with np.errstate(divide="ignore"):
                lead = np.floor(np.log2(np.where(ay > 0, ay, 1.0)))
            half_step = np.where(ay >= 2.0 ** -6, 2.0 ** (lead - 4), 2.0 ** -10)
            # the fp32 allowance of y: that of p', plus the scale's own rounding
            allow = (PR.TOL * np.maximum(np.abs(ref["p"]), fl["p"]) + 2.0 ** -23 * np.abs(ref["p"])) * sc
            judged = allow < half_step
            far = judged & (np.abs(_monotone_e4m3(got) - _monotone_e4m3(q_ref)) > 1)
            assert not far.any(), (f"tensor {i} t={t}: {far.sum()} codes more than one step from the "
                                   f"double-precision code, first at {np.flatnonzero(far)[:5]}")
            differ += int(np.count_nonzero(got != q_ref))
            judged_total += int(judged.sum())
    print(f"fp8 codes against codes decided in double: {differ} of {3 * st.total:,} differ; "
          f"none of the {judged_total:,} judged is more than one step away", flush=True)
    st.close()
