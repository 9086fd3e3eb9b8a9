"""Pins of the oracle's reduce, AdamW and bf16 cast (CPU only).

Each pin checks the oracle against something other than itself: a closed form
of the update rule, a library routine (torch.optim.AdamW in float64, torch's
fp32->bf16 conversion, numpy.mean), hand-worked rounding cases, exact rational
arithmetic, or the sharded == unsharded equivalence the ZeRO state sharding
post measures between its sharded modes and plain DDP.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import layout as L
from oracle import step as O
from rank_step_amd.workloads import HPARAMS

HP = dict(HPARAMS)
LR, B1, B2, EPS, WD = HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], HP["weight_decay"]


# ----------------------------------------------------------------- reduce

def test_reduce_identical_slices_exact():
    # With 8-bit significands (bf16 values) every partial sum of up to 16
    # copies is exact in float64, so the mean must return the slice exactly.
    rng = np.random.default_rng(0)
    x = np.ldexp(np.round(np.ldexp(rng.uniform(0.5, 1, 1000), 8)), rng.integers(-30, 30, 1000) - 8)
    x *= np.where(rng.random(1000) < 0.5, -1.0, 1.0)
    for N in (1, 2, 3, 4, 5, 8, 16):
        assert np.array_equal(O.reduce_mean(np.stack([x] * N)), x)


def test_reduce_antisymmetric_is_zero():
    # 8-bit significands within a 20-binade spread: all partial sums are exact,
    # so slices with x_q = -x_{N-1-q} must reduce to exactly +0.
    rng = np.random.default_rng(1)
    for N in (2, 4, 6, 8):
        mant = np.round(np.ldexp(rng.uniform(0.5, 1, (N // 2, 257)), 8))
        half = np.ldexp(mant, rng.integers(-10, 10, (N // 2, 257)) - 8)
        half *= np.where(rng.random((N // 2, 257)) < 0.5, -1.0, 1.0)
        sl = np.concatenate([half, -half[::-1]])      # x_q = -x_{N-1-q}
        g = O.reduce_mean(sl)
        assert np.all(g == 0.0)


def test_reduce_matches_numpy_mean():
    rng = np.random.default_rng(2)
    for N in (1, 3, 4, 5, 8, 32):
        sl = rng.standard_normal((N, 4096)) * 10.0 ** rng.uniform(-6, 2, (N, 4096))
        ref = np.mean(sl, axis=0)
        got = O.reduce_mean(sl)
        scale = np.mean(np.abs(sl), axis=0)
        assert np.all(np.abs(got - ref) <= 4 * N * np.finfo(np.float64).eps * scale)


def test_reduce_widening_exact():
    # bf16 bit patterns widen to exactly the float32 with the same top half
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    w = O.widen_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(w), nan)
    assert np.array_equal(w[~nan], ref[~nan])


# ----------------------------------------------------------------- AdamW

def test_step1_closed_form():
    # m = v = 0 at t = 1: mhat = G, vhat = G^2, so p' = p(1 - lr wd) - lr G / (|G| + eps)
    G = np.concatenate([np.logspace(-12, 2, 4001), -np.logspace(-12, 2, 4001)])
    p = np.linspace(-1.0, 1.0, G.size)
    z = np.zeros_like(G)
    pn, mn, vn = O.adamw(p, z, z, G, 1, LR, B1, B2, EPS, WD)
    ref = p * (1 - LR * WD) - LR * G / (np.abs(G) + EPS)
    assert np.max(np.abs(pn - ref) / (np.abs(p) + LR)) <= 1e-14
    # about lr * sign(G) for |G| >> eps, lr / 2 at |G| = eps
    big = np.abs(G) > 1e-4
    upd = p * (1 - LR * WD) - pn
    assert np.allclose(upd[big], LR * np.sign(G[big]), rtol=1e-4, atol=0)
    _, _, _ = O.adamw(np.zeros(1), np.zeros(1), np.zeros(1), np.array([EPS]), 1, LR, B1, B2, EPS, WD)
    pe, _, _ = O.adamw(np.zeros(1), np.zeros(1), np.zeros(1), np.array([EPS]), 1, LR, B1, B2, EPS, WD)
    assert abs(pe[0] + LR / 2) <= 1e-17


def test_zero_gradient_pure_decay():
    rng = np.random.default_rng(3)
    p0 = rng.standard_normal(512)
    p, m, v = p0.copy(), np.zeros(512), np.zeros(512)
    for t in range(1, 11):
        p, m, v = O.adamw(p, m, v, np.zeros(512), t, LR, B1, B2, EPS, WD)
        assert np.all(m == 0) and np.all(v == 0)
        ref = p0 * (1 - LR * WD) ** t
        assert np.max(np.abs(p - ref) / np.abs(ref)) <= 1e-14


def test_constant_gradient_closed_form():
    # constant G: mhat = G and vhat = G^2 at every t, so with c = 1 - lr wd,
    # p_t = c^t p0 - u (1 - c^t) / (1 - c), u = lr G / (|G| + eps)
    rng = np.random.default_rng(4)
    G = rng.standard_normal(300) * 10.0 ** rng.uniform(-9, 1, 300)
    p0 = rng.standard_normal(300) * 0.02
    c = 1 - LR * WD
    u = LR * G / (np.abs(G) + EPS)
    p, m, v = p0.copy(), np.zeros(300), np.zeros(300)
    for t in range(1, 21):
        p, m, v = O.adamw(p, m, v, G, t, LR, B1, B2, EPS, WD)
        # 1 - c^t and c^t without cancellation
        one_minus_ct = -np.expm1(t * np.log1p(-LR * WD))
        ref = (1 - one_minus_ct) * p0 - u * one_minus_ct / (LR * WD)
        scale = np.abs(c ** t * p0) + np.abs(u) * t
        assert np.max(np.abs(p - ref) / scale) <= 1e-13, t


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_adamw_float64(seed):
    # The reading taken is torch.optim.AdamW; its float64 CPU path is the library pin.
    rng = np.random.default_rng(10 + seed)
    n = 2000
    p0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * 10.0 ** rng.uniform(-8, 0, n) for _ in range(8)]
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=LR, betas=(B1, B2), eps=EPS, weight_decay=WD,
                            foreach=False, fused=False)
    p, m, v = p0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = O.adamw(p, m, v, g, t, LR, B1, B2, EPS, WD)
        st = opt.state[tp]
        for mine, theirs in ((p, tp.detach()), (m, st["exp_avg"]), (v, st["exp_avg_sq"])):
            theirs = theirs.numpy()
            assert np.max(np.abs(mine - theirs) / (np.abs(theirs) + 1e-300)) <= 1e-12


# ----------------------------------------------------------------- bf16 cast

def test_bf16_golden_cases():
    d = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.json")))
    xs = np.array([c["sign"] * c["mant"] * 2.0 ** c["exp2"] for c in d["cases"]])
    got = O.bf16_rne(xs)
    for c, b in zip(d["cases"], got):
        assert int(b) == int(c["bits"], 16), c["what"]


def test_bf16_specials():
    got = O.bf16_rne(np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0]))
    assert list(map(int, got)) == [0x7FC0, 0xFFC0, 0x7F80, 0xFF80, 0x0000, 0x8000]


def test_bf16_fp32_inputs_match_torch():
    # torch's fp32 -> bf16 conversion rounds to nearest even; for every non-NaN
    # fp32 input the oracle must agree bit for bit.
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF,
                        0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x00000001, 0x00008000,
                        0x00018000, 0x3F808000, 0x3F818000, 0x3F807FFF], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    # every rounding boundary pattern of the low half, with random top halves
    low = np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32)
    tops = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32) << np.uint32(16)
    bits = np.concatenate([bits, (tops[:, None] | low[None, :]).ravel()])
    f = bits.view(np.float32)
    keep = ~np.isnan(f)
    f = f[keep]
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_rne(f.astype(np.float64))
    assert np.array_equal(got, ref)


def _bf16_value(b):
    b = int(b)
    s = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if e == 0:
        return s * Fraction(f, 1 << 7) * Fraction(1, 1 << 126)
    return s * (1 + Fraction(f, 1 << 7)) * (Fraction(2) ** (e - 127))


def test_bf16_double_inputs_nearest_even_exact():
    # brute force against the definition with exact rationals: the result is the
    # nearer of its two bf16 neighbours, and on a tie its last bit is even.
    rng = np.random.default_rng(6)
    x = rng.standard_normal(3000) * 10.0 ** rng.uniform(-40, 38, 3000)
    # force ties and near-ties: bf16 midpoints nudged by tiny amounts
    mids = []
    for b in rng.integers(0x0001, 0x7F7F, 500):
        lo, hi = _bf16_value(b), _bf16_value(b + 1)
        mid = (lo + hi) / 2
        for d in (Fraction(0), Fraction(1, 1 << 60), -Fraction(1, 1 << 60)):
            mids.append(float(mid + d * mid))
    x = np.concatenate([x, np.array(mids)])
    got = O.bf16_rne(x)
    for xi, b in zip(x, got):
        X = Fraction(float(xi))
        v = _bf16_value(b)
        mag = int(b) & 0x7FFF
        if mag == 0x7F80:
            assert abs(X) >= (Fraction(2) - Fraction(1, 256)) * Fraction(2) ** 127
            continue
        nb = [mag - 1, mag + 1] if mag > 0 else [1]
        for n in nb:
            other = _bf16_value((int(b) & 0x8000) | n)
            if abs(X - other) < abs(X - v):
                raise AssertionError((xi, hex(int(b))))
            if abs(X - other) == abs(X - v):
                assert (mag & 1) == 0


# ----------------------------------------------------------------- whole rank step

def test_padding_stays_zero_with_garbage_inputs():
    rng = np.random.default_rng(7)
    S, valid, N = 37, 29, 3
    p = rng.standard_normal(S)
    p[valid:] = 1e30
    m = rng.standard_normal(S) ** 2
    v = rng.standard_normal(S) ** 2
    m[valid:] = np.nan
    v[valid:] = np.inf
    sl = rng.standard_normal((N, S))
    sl[:, valid:] = np.nan
    for t in (1, 2, 3):
        out = O.rank_step(p, m, v, sl, valid, t, HP)
        for k in ("g", "p", "m", "v"):
            assert np.all(out[k][valid:] == 0.0) and not np.any(np.signbit(out[k][valid:]))
        assert np.all(out["bf16"][valid:] == 0)
        p, m, v = out["p"], out["m"], out["v"]
    out = O.rank_step(p, m, v, sl, 0, 4, HP)       # valid = 0: an all-padding rank
    assert all(np.all(out[k] == 0.0) for k in ("g", "p", "m", "v"))


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 8])
def test_sharded_equals_unsharded(N):
    # Concatenating all N rank-shard results (pad stripped) is bitwise equal to
    # one unsharded AdamW step on the mean of the N full gradients.
    rng = np.random.default_rng(100 + N)
    for P in list(range(0, 65)):
        numels = [P // 3, P - P // 3 - P // 4, P // 4]
        p0 = rng.standard_normal(P) * 0.02
        m0 = rng.standard_normal(P) * 1e-3
        v0 = np.abs(rng.standard_normal(P)) * 1e-6
        grads = rng.standard_normal((N, P)) * 1e-2     # rank q's full gradient
        t = int(rng.integers(1, 6))
        G = O.reduce_mean(grads)
        ref_p, ref_m, ref_v = O.adamw(p0, m0, v0, G, t, LR, B1, B2, EPS, WD)
        ref_b = O.bf16_rne(ref_p)

        cat = {k: [] for k in ("p", "m", "v", "bf16")}
        for r in range(N):
            _, S, _, valid = L.flat_layout(numels, N, r)
            lo = r * S

            def shard(x, fill):
                out = np.full(S, fill, dtype=np.float64)
                out[:valid] = x[lo:lo + valid]
                return out
            # garbage in every pad position: the step must neither read nor keep it
            sl = np.stack([shard(grads[q], np.nan) for q in range(N)])
            out = O.rank_step(shard(p0, 7.0), shard(m0, -3.0), shard(v0, np.inf), sl, valid, t, HP)
            for k in cat:
                cat[k].append(out[k][:valid])
                assert np.all(out[k][valid:] == 0)
        for k, ref in (("p", ref_p), ("m", ref_m), ("v", ref_v), ("bf16", ref_b)):
            got = np.concatenate(cat[k]) if cat[k] else np.zeros(0)
            assert np.array_equal(got, ref), (P, k)
