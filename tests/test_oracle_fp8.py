"""Pins of the oracle's fp8 (OCP E4M3, "e4m3fn") quantisation (CPU only):
every one of the 256 codes round-trips, every midpoint between neighbouring
codes ties to the even code, torch's float8_e4m3fn conversion (a library
routine) agrees on in-range fp32 inputs, saturation at 448, and mutants that
must be caught."""

import numpy as np
import pytest
import torch

from oracle import fp8 as F


def _finite_codes():
    c = np.arange(256, dtype=np.int64)
    return c[(c & 0x7F) != 0x7F].astype(np.uint8)


def test_value_table_landmarks():
    v = F.e4m3_value(np.array([0x7E, 0x08, 0x01, 0x38, 0x00, 0x80, 0xFE, 0x7F], dtype=np.uint8))
    assert v[0] == 448.0 and v[1] == 2.0 ** -6 and v[2] == 2.0 ** -9 and v[3] == 1.0
    assert v[4] == 0.0 and v[5] == 0.0 and np.signbit(v[5]) and v[6] == -448.0 and np.isnan(v[7])


def test_every_code_round_trips():
    c = _finite_codes()
    assert np.array_equal(F.e4m3_rne(F.e4m3_value(c)), c)
    assert F.e4m3_rne(np.array([np.nan]))[0] == 0x7F
    assert F.e4m3_rne(np.array([-np.nan]))[0] == 0xFF


def test_midpoints_tie_to_even():
    c = np.arange(0x00, 0x7E, dtype=np.int64)                 # positive codes with a finite successor
    lo, hi = F.e4m3_value(c.astype(np.uint8)), F.e4m3_value((c + 1).astype(np.uint8))
    mid = (lo + hi) / 2                                         # exact in float64
    got = F.e4m3_rne(mid).astype(np.int64)
    assert np.array_equal(got, np.where(c % 2 == 0, c, c + 1))
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(F.e4m3_rne(mid - eps).astype(np.int64), c)
    assert np.array_equal(F.e4m3_rne(mid + eps).astype(np.int64), c + 1)
    assert np.array_equal(F.e4m3_rne(-mid).astype(np.int64), np.where(c % 2 == 0, c, c + 1) | 0x80)


def test_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(200000) * 10.0 **
                        rng.uniform(-5, 2, 200000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_rne(x.astype(np.float64)), ref)


def test_quantize_saturates_and_scales():
    s = F.scale_of(2.0)
    assert s == np.float32(224.0)
    q = F.quantize(np.array([2.0, -2.0, 1.0, 3.0, 1e30, -np.inf, np.nan], dtype=np.float32), s)
    assert list(q[:5]) == [0x7E, 0xFE, F.e4m3_rne(np.array([224.0]))[0], 0x7E, 0x7E]
    assert q[5] == 0xFE and (q[6] & 0x7F) == 0x7F
    assert F.scale_of(0.0) == np.float32(448.0) / np.float32(1e-12)
    assert np.isnan(F.scale_of(np.nan))
    # |q value / scale - p| <= half a code spacing relative, for in-range values
    rng = np.random.default_rng(1)
    p = (rng.standard_normal(10000) * 0.02).astype(np.float32)
    sc = F.scale_of(F.amax(p))
    back = F.e4m3_value(F.quantize(p, sc)) / np.float64(sc)
    rel = np.abs(back - p) / np.maximum(np.abs(p), 2.0 ** -6 / np.float64(sc))
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_amax_propagates_nan():
    assert F.amax(np.array([1.0, -3.0, 2.0])) == 3.0
    assert np.isnan(F.amax(np.array([1.0, np.nan])))
    assert F.amax(np.zeros(0)) == 0.0


_RNE = F.e4m3_rne


def _trunc(x):
    x = np.asarray(x, dtype=np.float64)
    r = _RNE(x)
    v = F.e4m3_value(r)
    over = np.abs(v) > np.abs(x)
    return np.where(over & (r & 0x7F > 0), r - 1, r).astype(np.uint8)


def _quantize_no_saturation(p, scale):
    y = (np.asarray(p, dtype=np.float32) * np.float32(scale)).astype(np.float64)
    r = _RNE(np.clip(y, -448, 448))
    return np.where(np.abs(y) > 448, 0x7F, r).astype(np.uint8)       # out of range -> NaN


@pytest.mark.parametrize("attr,mut", [("e4m3_rne", _trunc), ("quantize", _quantize_no_saturation)])
def test_mutants_are_caught(attr, mut, monkeypatch):
    monkeypatch.setattr(F, attr, mut)
    caught = 0
    for pin in (test_every_code_round_trips, test_midpoints_tie_to_even, test_matches_torch_in_range,
                test_quantize_saturates_and_scales):
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught += 1
    assert caught >= 1
