"""Pins of the oracle's gradient accumulation (CPU only): with values whose
sums are exact (8-bit significands in a narrow range) the synchronised and
no_sync paths agree bit for bit and equal the closed form; with general values
they agree within rounding; and mutants are caught."""

import numpy as np
import pytest

from oracle import accum as A
from oracle import step as O


def _exact_values(rng, shape):
    m = np.round(np.ldexp(rng.uniform(0.5, 1, shape), 8))
    return np.ldexp(m, rng.integers(-6, 6, shape) - 8) * np.where(rng.random(shape) < 0.5, -1, 1)


@pytest.mark.parametrize("N,K", [(1, 1), (2, 3), (4, 4), (8, 2), (16, 5)])   # N a power of two: exact division
def test_paths_agree_exactly_on_exact_values(N, K):
    rng = np.random.default_rng(10 * N + K)
    micro = [_exact_values(rng, (N, 300)) for _ in range(K)]
    a, b = A.synchronised(micro), A.no_sync(micro)
    assert np.array_equal(a, b)
    ref = np.sum(np.stack(micro), axis=(0, 1)) / N          # exact here
    assert np.array_equal(a, ref)


def test_constant_micro_batches_closed_form():
    N, K, c = 4, 6, 0.375
    micro = [np.full((N, 50), c) for _ in range(K)]
    assert np.all(A.synchronised(micro) == K * c)
    assert np.all(A.no_sync(micro) == K * c)


def test_paths_agree_within_rounding():
    rng = np.random.default_rng(3)
    N, K = 8, 4
    micro = [rng.standard_normal((N, 5000)) * 1e-3 for _ in range(K)]
    a, b = A.synchronised(micro), A.no_sync(micro)
    scale = np.sum(np.abs(np.stack(micro)), axis=(0, 1)) / N
    assert np.all(np.abs(a - b) <= 8 * (N + K) * 2.3e-16 * scale)


def test_first_micro_batch_is_a_copy():
    x = np.array([-0.0, 1.5, -2.25])
    got = A.accumulate(None, x)
    assert np.array_equal(got, x) and np.signbit(got[0])


def test_mutants_are_caught(monkeypatch):
    def forgets_first(acc, micro):          # first micro-batch dropped
        return np.zeros_like(np.asarray(micro, dtype=np.float64)) if acc is None else acc + micro

    def averages_micro(slices_per_micro):   # divides by the micro-batch count too
        return sum(O.reduce_mean(s) for s in slices_per_micro) / len(slices_per_micro)
    for attr, fn in (("accumulate", forgets_first), ("synchronised", averages_micro)):
        with monkeypatch.context() as mp:
            mp.setattr(A, attr, fn)
            caught = 0
            for pin in (lambda: test_paths_agree_exactly_on_exact_values(2, 3),
                        test_constant_micro_batches_closed_form):
                try:
                    pin()
                except AssertionError:
                    caught += 1
            assert caught >= 1, attr
