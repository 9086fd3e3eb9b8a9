"""The oracle's pins must catch plausible mistakes: each mutant below plants one
in a copy of the oracle's arithmetic (on the CPU) and at least one pin has to
fail against it."""

import numpy as np
import pytest

from oracle import step as O
import tests.test_oracle_step as pins

ADAMW_PINS = [pins.test_step1_closed_form, pins.test_zero_gradient_pure_decay,
              pins.test_constant_gradient_closed_form,
              lambda: pins.test_matches_torch_adamw_float64(0)]


def _mk(kind):
    def adamw(p, m, v, g, t, lr, b1, b2, eps, wd):
        p, m, v, g = (np.asarray(a, dtype=np.float64) for a in (p, m, v, g))
        decay = 1.0 - (wd if kind == "wd_not_scaled_by_lr" else lr * wd)
        m2 = b1 * m + (1 - b1) * g
        v2 = b2 * v + (1 - b2) * (g if kind == "v_uses_g_not_g2" else g * g)
        tt = t - 1 if kind == "bias_correction_off_by_one" else t
        bc1 = 1.0 if kind == "no_bias_correction_m" else 1 - b1 ** max(tt, 1)
        bc2 = 1.0 if kind == "no_bias_correction_v" else 1 - b2 ** max(tt, 1)
        if kind == "bias_correction_off_by_one" and t == 1:
            bc1 = bc2 = 1.0
        if kind == "eps_inside_sqrt":
            den = np.sqrt(v2 / bc2 + eps)
        elif kind == "eps_before_bias_correction":
            den = (np.sqrt(v2) + eps) / np.sqrt(bc2)
        else:
            den = np.sqrt(v2 / bc2) + eps
        upd = lr * (m2 / bc1) / den
        if kind == "decay_after_update":
            return (p - upd) * decay, m2, v2
        if kind == "decay_on_gradient":     # L2 penalty instead of decoupled decay
            g2 = g + wd * p
            return adamw_l2(p, m, v, g2, t, lr, b1, b2, eps)
        if kind == "update_sign_flipped":
            return p * decay + upd, m2, v2
        return p * decay - upd, m2, v2

    def adamw_l2(p, m, v, g, t, lr, b1, b2, eps):
        m2 = b1 * m + (1 - b1) * g
        v2 = b2 * v + (1 - b2) * g * g
        return p - lr * (m2 / (1 - b1 ** t)) / (np.sqrt(v2 / (1 - b2 ** t)) + eps), m2, v2
    return adamw


MUTANTS = ["wd_not_scaled_by_lr", "v_uses_g_not_g2", "bias_correction_off_by_one",
           "no_bias_correction_m", "no_bias_correction_v", "eps_inside_sqrt",
           "eps_before_bias_correction", "decay_after_update", "decay_on_gradient",
           "update_sign_flipped"]


def test_unmutated_passes(monkeypatch):
    monkeypatch.setattr(O, "adamw", _mk("none"))
    for pin in ADAMW_PINS:
        pin()


@pytest.mark.parametrize("kind", MUTANTS)
def test_adamw_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(O, "adamw", _mk(kind))
    caught = 0
    for pin in ADAMW_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


def _rne_truncate(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rne_half_up(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x8000) >> 16).astype(np.uint16)


def _rne_via_fp32(x):
    # double rounding: double -> fp32 -> bf16
    f = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return r.astype(np.uint16)


@pytest.mark.parametrize("mut", [_rne_truncate, _rne_half_up, _rne_via_fp32])
def test_cast_mutant_is_caught(mut, monkeypatch):
    monkeypatch.setattr(O, "bf16_rne", mut)
    caught = 0
    for pin in (pins.test_bf16_golden_cases, pins.test_bf16_specials,
                pins.test_bf16_fp32_inputs_match_torch,
                pins.test_bf16_double_inputs_nearest_even_exact):
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, Exception):
            caught += 1
    assert caught >= 1


def test_reduce_mutants_are_caught(monkeypatch):
    def sum_not_mean(x):
        return np.sum(np.asarray(x, dtype=np.float64), axis=0)

    def drops_last(x):
        x = np.asarray(x, dtype=np.float64)
        return np.sum(x[:-1], axis=0) / x.shape[0] if x.shape[0] > 1 else x[0]
    for mut in (sum_not_mean, drops_last):
        monkeypatch.setattr(O, "reduce_mean", mut)
        caught = 0
        for pin in (pins.test_reduce_identical_slices_exact, pins.test_reduce_antisymmetric_is_zero,
                    pins.test_reduce_matches_numpy_mean):
            try:
                pin()
            except AssertionError:
                caught += 1
        assert caught >= 1
