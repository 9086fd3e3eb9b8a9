"""Pins of the oracle's gradient-norm clipping (CPU only): torch's
clip_grad_norm_ in float64 (the library routine the page names), the closed
form for a constant gradient, shard-wise == unsharded squared norms (within
the rounding of the N per-rank partial sums), and mutants that must be caught."""

import math

import numpy as np
import pytest
import torch

from oracle import clip as C
from oracle import layout as L
from oracle import step as O
from rank_step_amd.workloads import HPARAMS


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("max_norm", [0.05, 1.0, 1e9])
def test_matches_torch_clip_grad_norm(seed, max_norm):
    rng = np.random.default_rng(seed)
    grads = [rng.standard_normal(rng.integers(1, 3000)) * 10.0 ** rng.uniform(-4, 0) for _ in range(5)]
    params = [torch.nn.Parameter(torch.zeros(len(g), dtype=torch.float64)) for g in grads]
    for p, g in zip(params, grads):
        p.grad = torch.from_numpy(g.copy())
    tnorm = float(torch.nn.utils.clip_grad_norm_(params, max_norm, norm_type=2.0, foreach=False))
    norm, coef = C.clip_coef([C.sq_norm(g) for g in grads], max_norm)
    assert abs(norm - tnorm) <= 1e-14 * tnorm
    for p, g in zip(params, grads):
        assert np.allclose(g * coef, p.grad.numpy(), rtol=1e-14, atol=0)


def test_constant_gradient_closed_form():
    for P, c in ((1, 3.0), (1000, -0.25), (12345, 1e-3)):
        norm, coef = C.clip_coef([C.sq_norm(np.full(P, c))], 1.0)
        assert abs(norm - abs(c) * math.sqrt(P)) <= 2e-16 * norm
        assert coef == (1.0 if norm <= 1.0 - 1e-6 else 1.0 / (norm + 1e-6))


def test_coef_properties():
    assert C.clip_coef([0.0], 1.0) == (0.0, 1.0)               # zero gradient: no scaling
    n, c = C.clip_coef([4.0], 1.0)                             # norm 2 -> coef 1/(2+1e-6)
    assert n == 2.0 and abs(c * (2.0 + 1e-6) - 1.0) < 1e-15
    n, c = C.clip_coef([float("inf")], 1.0)
    assert n == float("inf") and c == 0.0
    n, c = C.clip_coef([float("nan")], 1.0)
    assert math.isnan(n) and math.isnan(c)


@pytest.mark.parametrize("N", [1, 2, 3, 4, 8])
def test_sharded_sq_norm_equals_unsharded(N):
    rng = np.random.default_rng(N)
    for P in (0, 1, 7, 63, 64, 1000):
        numels = [P // 2, P - P // 2]
        grads = rng.standard_normal((N, P)) * 1e-2
        G = O.reduce_mean(grads)
        full = C.sq_norm(G)
        parts = []
        for r in range(N):
            _, S, _, valid = L.flat_layout(numels, N, r)
            parts.append(C.sq_norm(G[r * S:r * S + valid]))
        # each per-rank partial is correctly rounded once: N half-ulps at most
        assert abs(math.fsum(parts) - full) <= N * 2.3e-16 * full
        n1, c1 = C.clip_coef(parts, 0.1)
        n2, c2 = C.clip_coef([full], 0.1)
        assert abs(n1 - n2) <= N * 2.3e-16 * n2 and abs(c1 - c2) <= N * 4.5e-16 * c2


def test_clipped_rank_step_scales_gradient():
    rng = np.random.default_rng(9)
    S = 500
    p, m, v = rng.standard_normal(S) * 0.02, np.zeros(S), np.zeros(S)
    sl = rng.standard_normal((4, S)) * 1e-2
    a = O.rank_step(p, m, v, sl, S, 1, HPARAMS, grad_scale=0.5)
    b = O.rank_step(p, m, v, sl * 0.5, S, 1, HPARAMS)       # scaling slices by 1/2 is exact
    for k in ("p", "m", "v"):
        assert np.array_equal(a[k], b[k])


def _abs_sum(g):
    return math.fsum(np.abs(np.asarray(g, dtype=np.float64)).ravel().tolist())


def test_mutants_are_caught(monkeypatch):
    pins = [lambda: test_matches_torch_clip_grad_norm(0, 0.05), test_constant_gradient_closed_form,
            test_coef_properties]
    muts = {
        "abs_not_square": ("sq_norm", _abs_sum),
        "no_eps": ("clip_coef", lambda sq, mx: (math.sqrt(math.fsum(sq)), min(1.0, mx / math.sqrt(math.fsum(sq))) if math.fsum(sq) else 1.0)),
        "not_clamped": ("clip_coef", lambda sq, mx: (math.sqrt(math.fsum(sq)), mx / (math.sqrt(math.fsum(sq)) + 1e-6))),
        "no_sqrt": ("clip_coef", lambda sq, mx: (math.fsum(sq), min(1.0, mx / (math.fsum(sq) + 1e-6)))),
    }
    for name, (attr, fn) in muts.items():
        with monkeypatch.context() as mp:
            mp.setattr(C, attr, fn)
            caught = 0
            for pin in pins:
                try:
                    pin()
                except (AssertionError, ZeroDivisionError, ValueError):
                    caught += 1
            assert caught >= 1, name
