"""Comparison helpers for the GPU parity tests (test-side only).

The fp32 criterion is the mixed one: for each fp32 output x,

    |x_gpu - x_ref| <= TOL * max(|x_ref|, s_x)

where s_x is the magnitude of the terms that form x, so that cancellation
(a result much smaller than its terms) is judged against the terms' size:

    s_G = mean_q |x_q|                               reduced gradient
    s_m = beta1*|m| + (1-beta1)*s_G                  first moment
    s_v = beta2*v + (1-beta2)*s_G^2                  second moment
    s_p = |p|*(1-lr*wd) + lr*(s_m/bc1)/(sqrt(vhat)+eps) + d_p   parameter

d_p (only with ``widen=True``) carries the allowed error of G through the
denominator: G's allowance moves vhat by dvhat = (1-beta2)*2*|G|*s_G/bc2, and
the update lr*mhat/(sqrt(vhat)+eps) by
lr*|mhat|*dvhat / (2*sqrt(vhat)*(sqrt(vhat)+eps)^2) (first order).  It
matters where G cancels across many slices and v is tiny beside m, so that
the update hangs on a few bits of G: the tests that draw N = 33 slices or a
random N widen the floor with it; every other case is judged without it.

The inputs of the oracle are the GPU's own state before the step, widened
exactly (per-step resynchronisation), so one step's rounding is judged.
bf16: bit-exact to RNE of the GPU's own fp32 result, and within 1 ulp of RNE
of the oracle's result wherever the fp32 error allowance is below half a bf16
ulp of the value.
"""

import numpy as np
import torch

from oracle import step as O

TOL = 2e-6


def f64(t):
    return t.detach().to("cpu").numpy().astype(np.float64)


def bf16_bits(t):
    return t.detach().to("cpu").view(torch.int16).numpy().view(np.uint16)


def widen_slices(t, dtype):
    """[N, n] device slices -> float64 host array, exactly."""
    if dtype == "bf16":
        return O.widen_bf16_bits(bf16_bits(t))
    return t.detach().to("cpu").numpy().astype(np.float64)


def _denominator_term(ref, sl, sG, hp, t):
    """d_p above: the update's sensitivity to G's allowance through vhat.
    ``sl`` are the slices as the update sees them (already scaled by a clip
    coefficient), so their mean is the G the update uses."""
    lr, b1, b2, eps = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"]
    bc1 = 1 - b1 ** t
    bc2 = 1 - b2 ** t
    sq = np.sqrt(ref["v"] / bc2)
    g = np.mean(sl, axis=0) if sl.shape[0] else np.zeros(0)
    dvhat = (1 - b2) * 2 * np.abs(g) * sG / bc2
    mhat = np.abs(ref["m"]) / bc1
    with np.errstate(divide="ignore", invalid="ignore"):
        d = lr * mhat * dvhat / (2 * sq * (sq + eps) ** 2)
    return np.where(sq > 0, d, 0.0)


def floors(p, m, v, sl, ref, hp, t, widen=False):
    lr, b1, b2, eps, wd = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]
    sG = np.mean(np.abs(sl), axis=0) if sl.shape[0] else np.zeros(0)
    s_m = b1 * np.abs(m) + (1 - b1) * sG
    s_v = b2 * v + (1 - b2) * sG * sG
    bc1 = 1 - b1 ** t
    bc2 = 1 - b2 ** t
    vhat = ref["v"] / bc2
    s_p = np.abs(p) * (1 - lr * wd) + lr * (s_m / bc1) / (np.sqrt(vhat) + eps)
    if widen:
        s_p = s_p + _denominator_term(ref, sl, sG, hp, t)
    return {"g": sG, "m": s_m, "v": s_v, "p": s_p}


def free_floors(prev, sl, ref, hp, t, widen=False):
    """Floors for a free-running comparison: the term magnitudes carried along
    the whole trajectory, so that slack allowed at an earlier step (e.g. an
    element whose mean gradient cancelled to about eps) is still allowed.
    ``prev`` holds the previous step's floors (initially |p0|, |m0|, v0)."""
    lr, b1, b2, eps, wd = hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["weight_decay"]
    sG = np.mean(np.abs(sl), axis=0)
    s_m = b1 * prev["m"] + (1 - b1) * sG
    s_v = b2 * prev["v"] + (1 - b2) * sG * sG
    vhat = ref["v"] / (1 - b2 ** t)
    s_p = prev["p"] * (1 - lr * wd) + lr * (s_m / (1 - b1 ** t)) / (np.sqrt(vhat) + eps)
    if widen:
        s_p = s_p + _denominator_term(ref, sl, sG, hp, t)
    return {"g": sG, "m": s_m, "v": s_v, "p": s_p}


def assert_close(name, got, ref, floor, tol=TOL, abs_tol=0.0):
    """``abs_tol`` adds an absolute allowance: used only where results lie in
    fp32's subnormal range, whose spacing 2**-149 is coarser than any
    relative bound there."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bad_nan = np.isnan(got) != np.isnan(ref)
    assert not bad_nan.any(), f"{name}: NaN mismatch at {np.flatnonzero(bad_nan)[:5]}"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), f"{name}: infinity mismatch"
    ok = ~np.isnan(ref) & ~inf
    err = np.abs(got[ok] - ref[ok])
    lim = tol * np.maximum(np.abs(ref[ok]), floor[ok]) + abs_tol
    bad = err > lim
    if bad.any():
        i = np.flatnonzero(ok)[np.flatnonzero(bad)[:5]]
        raise AssertionError(f"{name}: {bad.sum()} of {ok.sum()} elements beyond tolerance; "
                             f"first at {i.tolist()}: got {got[i].tolist()} ref {ref[i].tolist()} "
                             f"floor {floor[i].tolist()}")
    # plain relative error where the result is not a cancellation
    big = np.abs(ref[ok]) >= 1e-3 * floor[ok]
    rel = err[big] / np.maximum(np.abs(ref[ok][big]), 1e-300)
    return float(rel.max()) if rel.size else 0.0


def mixed_ratio(got, ref, floor, tol=TOL):
    """Largest err / (tol * max(|ref|, floor)) over the finite results: the
    share of the mixed allowance the worst element uses (<= 1 passes)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ok = np.isfinite(ref) & np.isfinite(got)
    if not ok.any():
        return 0.0
    lim = tol * np.maximum(np.abs(ref[ok]), floor[ok])
    err = np.abs(got[ok] - ref[ok])
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(lim > 0, err / lim, np.where(err > 0, np.inf, 0.0))
    return float(r.max())


def literal_count(got, ref, tol=TOL):
    """Finite results outside the literal relative bound |err| <= tol*|ref|
    (those the mixed criterion admits through its floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ok = np.isfinite(ref)
    return int(np.count_nonzero(np.abs(got[ok] - ref[ok]) > tol * np.abs(ref[ok])))


def check_bf16(name, got_bits, gpu_p, ref_p, floor_p, tol=TOL):
    """bf16 output: exact RNE of the GPU's fp32 value; <= 1 ulp from RNE(oracle)."""
    own = O.bf16_rne(np.asarray(gpu_p, dtype=np.float64))
    mism = got_bits != own
    assert not mism.any(), (f"{name}: bf16 differs from RNE of its own fp32 at "
                            f"{np.flatnonzero(mism)[:5].tolist()}")
    ref_bits = O.bf16_rne(np.asarray(ref_p, dtype=np.float64))
    fin = ~np.isnan(np.asarray(ref_p))
    a = got_bits.astype(np.int32)
    b = ref_bits.astype(np.int32)
    # signed-magnitude -> monotone integers
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    half_ulp = np.abs(np.asarray(ref_p, dtype=np.float64)) * 2.0 ** -9
    judged = fin & (tol * np.maximum(np.abs(ref_p), floor_p) < half_ulp)
    far = judged & (np.abs(a - b) > 1)
    assert not far.any(), f"{name}: bf16 more than 1 ulp from RNE(oracle) at {np.flatnonzero(far)[:5]}"
    return int((a != b).sum())


def check_pad_zero(name, arr, valid):
    a = np.asarray(arr)
    tail = a[valid:]
    if tail.dtype == np.uint16:
        assert np.all(tail == 0), f"{name}: pad not zero"
    else:
        assert np.all(tail.view(np.uint32 if tail.dtype == np.float32 else np.uint64) == 0), \
            f"{name}: pad not +0"


def pow_steps(b, t):
    """b**t by binary powering in double, the library's own sequence of
    products for the bias corrections (Python floats are IEEE doubles)."""
    r, x = 1.0, float(b)
    t = int(t)
    while t > 0:
        if t & 1:
            r = r * x
        x = x * x
        t >>= 1
    return r


def fp32_replica_step(p, m, v, x, valid, t, hp, grad_scale=None):
    """The kernel's fp32 operation sequence, replayed in numpy (test-side
    only; the oracle stays float64).  Sum of the slices in slice order,
    one division by N (a multiplication by 1/N when N is a power of two);
    then AdamW with the fused multiply-adds the kernel writes, each rounded
    once (the exact product plus the addend, in 64-bit extended precision,
    rounded to fp32), correctly rounded division and square root, no flush
    of subnormals.  ``grad_scale`` (fp32, the clip coefficient) multiplies the
    reduced gradient once, in fp32.  Returns fp32 p', m', v' over the first
    ``valid`` elements."""
    f32 = np.float32
    ld = np.longdouble
    N = x.shape[0]

    def fma(a, b, c):
        return (a.astype(ld) * b.astype(ld) + c.astype(ld)).astype(f32)

    xs = x[:, :valid].astype(f32)
    s = xs[0].copy()
    for q in range(1, N):
        s = (s + xs[q]).astype(f32)
    if N > 1:
        s = s * f32(1.0 / N) if N & (N - 1) == 0 else s / f32(N)
    g = s.astype(f32)
    if grad_scale is not None:
        g = (g * f32(grad_scale)).astype(f32)
    bc1 = 1.0 - pow_steps(hp["beta1"], t)
    bc2 = 1.0 - pow_steps(hp["beta2"], t)
    decay = f32(1.0 - hp["lr"] * hp["weight_decay"])
    b1, omb1 = f32(hp["beta1"]), f32(1.0 - hp["beta1"])
    b2, omb2 = f32(hp["beta2"]), f32(1.0 - hp["beta2"])
    step = f32(hp["lr"] / bc1)
    isb = f32(1.0 / np.sqrt(bc2))
    eps = f32(hp["eps"])
    p, m, v = (a[:valid].astype(f32) for a in (p, m, v))
    full = np.full(valid, 1, dtype=f32)
    p1 = (p * decay).astype(f32)
    mn = fma(b1 * full, m, (omb1 * g).astype(f32))
    vn = fma(b2 * full, v, (omb2 * (g * g).astype(f32)).astype(f32))
    den = fma(np.sqrt(vn).astype(f32), isb * full, eps * full)
    pn = fma(-step * full, (mn / den).astype(f32), p1)
    return pn, mn, vn
