"""The oracle's C step (oracle/rank_step.c) and the C parity checker
(tests/c/fullcheck.c), pinned on the CPU:

* the C step equals oracle.step bit for bit (g, p', m', v') over slice counts,
  slice dtypes, step counts and hyperparameters, with zeros of both signs,
  subnormals, huge values, NaN and infinities planted in every input;
* its bf16 rounding, and the checker's, equal oracle.step.bf16_rne bit for
  bit over every class of double (ties, subnormal bf16, the overflow edge,
  NaN, infinities);
* the checker's counts equal those tests/parity.py's rules give, on results
  with planted errors on both sides of the tolerance and planted wrong bf16
  words.
"""

import numpy as np
import pytest

from oracle import cstep as C
from oracle import step as O
from tests import fullcheck as FC
from tests import parity as PR

HP = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.01}


def _inputs(rng, n, N, sdt, special):
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.standard_normal(n) ** 2 * 1e-6).astype(np.float32)
    x = (rng.standard_normal((N, n)) * 1e-2).astype(np.float32)
    if special:
        vals = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 3e38, -3e38, np.inf, -np.inf, np.nan,
                         1.0, -1.0], dtype=np.float32)
        for a in (p, m, x.reshape(-1)):
            idx = rng.integers(0, a.size, 64)
            a[idx] = rng.choice(vals, 64)
        idx = rng.integers(0, n, 32)
        v[idx] = rng.choice(np.array([0.0, 1e-45, 1e-40, 3e38, np.inf, np.nan], dtype=np.float32), 32)
    if sdt == "bf16":
        raw = (x.view(np.uint32) >> 16).astype(np.uint16)
        wide = O.widen_bf16_bits(raw)
    else:
        raw = x
        wide = x.astype(np.float64)
    return p, m, v, raw, wide


def _same(a, b):
    nan = np.isnan(a)
    return np.array_equal(nan, np.isnan(b)) and np.array_equal(a[~nan].view(np.uint64),
                                                              b[~nan].view(np.uint64))


@pytest.mark.parametrize("sdt", ["bf16", "f32"])
@pytest.mark.parametrize("N", [1, 3, 4, 8, 33])
@pytest.mark.parametrize("special", [False, True])
def test_c_step_equals_numpy_oracle_bitwise(sdt, N, special):
    rng = np.random.default_rng(1000 * N + special)
    n = 5003
    p, m, v, raw, wide = _inputs(rng, n, N, sdt, special)
    hps = [HP, dict(HP, weight_decay=0.0), dict(HP, beta1=0.0, eps=0.0),
           {"lr": 0.37, "beta1": 0.5, "beta2": 0.25, "eps": 1e-3, "weight_decay": 1.5}]
    with np.errstate(all="ignore"):
        for hp in hps:
            for t in (1, 2, 7, 1000):
                got = C.rank_step(p, m, v, raw, sdt, t, hp)
                ref = O.rank_step(p.astype(np.float64), m.astype(np.float64), v.astype(np.float64),
                                  wide, n, t, hp)
                for k in ("g", "p", "m", "v"):
                    assert _same(got[k], ref[k]), (k, hp, t)
                # from a state held in double: a second step on the oracle's own results
                got2 = C.rank_step(ref["p"], ref["m"], ref["v"], raw, sdt, t + 1, hp)
                ref2 = O.rank_step(ref["p"], ref["m"], ref["v"], wide, n, t + 1, hp)
                for k in ("g", "p", "m", "v"):
                    assert _same(got2[k], ref2[k]), (k, hp, t + 1)


def test_c_bf16_rne_equals_numpy_oracle():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-45, 39, 20000),
        np.ldexp(rng.integers(1, 1 << 9, 4000).astype(np.float64) + 0.5, -141),   # ties, subnormal bf16
        np.ldexp(rng.integers(1 << 7, 1 << 8, 4000).astype(np.float64) + 0.5, -7),  # ties, normal
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, 3.3895313892515355e38,
                  3.3961775292304690e38, 3.4028234663852886e38, 1e300, -1e300, 5e-324, 2 ** -133,
                  2 ** -134, 1.5 * 2 ** -134, 2 ** -126, 2 ** -127]),
    ])
    with np.errstate(all="ignore"):
        want = O.bf16_rne(x)
        assert np.array_equal(C.bf16_rne(x), want)
        assert np.array_equal(FC.rne(x), want)      # the checker's own rounding


def _expected_counts(p0, m0, v0, wide, ref, gpu, bits, t):
    """Counts by the rules of tests/parity.py (assert_close, literal_count,
    mixed_ratio and check_bf16), computed with its numpy code."""
    fl = PR.floors(p0.astype(np.float64), m0.astype(np.float64), v0.astype(np.float64), wide, ref,
                   HP, t)
    out = {}
    for k in ("g", "p", "m", "v"):
        got = gpu[k].astype(np.float64)
        r = ref[k]
        lim = PR.TOL * np.maximum(np.abs(r), fl[k])
        out[k] = (int(np.count_nonzero(np.abs(got - r) > lim)), PR.literal_count(got, r),
                  PR.mixed_ratio(got, r, fl[k]))
    own = O.bf16_rne(gpu["p"].astype(np.float64))
    want = O.bf16_rne(ref["p"])
    a = bits.astype(np.int32)
    b = want.astype(np.int32)
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    judged = PR.TOL * np.maximum(np.abs(ref["p"]), fl["p"]) < np.abs(ref["p"]) * 2.0 ** -9
    out["bf16"] = (int(np.count_nonzero(bits != own)), int(np.count_nonzero(judged & (np.abs(a - b) > 1))),
                   int(np.count_nonzero(bits != want)))
    return out


@pytest.mark.parametrize("sdt,N,t", [("bf16", 8, 1), ("bf16", 8, 4), ("f32", 4, 2), ("f32", 1, 3)])
def test_checker_counts_match_parity_rules(sdt, N, t):
    rng = np.random.default_rng(31 * N + t)
    n = 40000
    p0, m0, v0, raw, wide = _inputs(rng, n, N, sdt, False)
    ref = C.rank_step(p0, m0, v0, raw, sdt, t, HP)
    gpu = {k: ref[k].astype(np.float32) for k in ("g", "p", "m", "v")}
    # planted errors: relative sizes well inside and well outside 2e-6, on
    # disjoint random elements of each output
    for k in ("g", "p", "m", "v"):
        idx = rng.permutation(n)[:600]
        f = np.concatenate([np.full(200, 1e-7), np.full(200, 5e-5), np.full(200, -3e-3)])
        gpu[k][idx] = (ref[k][idx] * (1.0 + f)).astype(np.float32)
    gpu["p"][rng.integers(0, n, 5)] = np.nan
    bits = O.bf16_rne(gpu["p"].astype(np.float64))
    bits[rng.integers(0, n, 40)] ^= np.uint16(1)        # one ulp off their own fp32
    bits[rng.integers(0, n, 40)] ^= np.uint16(0x40)     # far off
    with np.errstate(all="ignore"):
        want = _expected_counts(p0, m0, v0, wide, ref, gpu, bits, t)
    s = FC.check_block(0, p0, m0, v0, raw, sdt, t, HP, ref, gpu["p"], gpu["m"], gpu["v"],
                       gpu_g=gpu["g"], gpu_bf16=bits).as_dict()
    for k in ("g", "m", "v"):
        bad, lit, worst = want[k]
        assert s[k]["bad"] == bad and s[k]["literal"] == lit, (k, s[k], want[k])
        assert abs(s[k]["worst"] - worst) <= 1e-9 * worst, (k, s[k]["worst"], worst)
    # p': the planted NaNs count as bad too (NaN where the oracle has a value)
    bad, lit, worst = want["p"]
    assert s["p"]["bad"] == bad + int(np.count_nonzero(np.isnan(gpu["p"]))), (s["p"], want["p"])
    assert abs(s["p"]["worst"] - worst) <= 1e-9 * worst
    assert s["bf16"]["not_own"] == want["bf16"][0] and s["bf16"]["far"] == want["bf16"][1]
    assert s["bf16"]["diff_vs_oracle"] == want["bf16"][2]
    assert s["g"]["bad"] > 0 and s["bf16"]["far"] > 0      # the planted errors are seen


def test_checker_passes_the_oracle_against_itself():
    rng = np.random.default_rng(5)
    n = 20000
    p0, m0, v0, raw, _ = _inputs(rng, n, 8, "bf16", False)
    ref = C.rank_step(p0, m0, v0, raw, "bf16", 2, HP)
    gp = ref["p"].astype(np.float32)
    s = FC.check_block(10, p0, m0, v0, raw, "bf16", 2, HP, ref, gp, ref["m"].astype(np.float32),
                       ref["v"].astype(np.float32), gpu_g=ref["g"].astype(np.float32),
                       gpu_bf16=C.bf16_rne(gp.astype(np.float64)))
    d = FC.assert_ok("self", s, check_g=True)
    assert all(d[k]["worst"] <= 0.5 for k in ("g", "p", "m", "v"))
    assert d["bf16"]["diff_vs_oracle"] >= 0
