"""ctypes binding of tests/c/fullcheck.c: the checks of tests/parity.py
(mixed tolerance, literal-bound counts, bf16 rules) element by element in C,
for the tests that compare every element of a full-size rank shard with the
oracle.  The C library is built by ``__graft_entry__.build()``; a missing
library is an error.
"""

import ctypes
import os

import numpy as np

from tests import parity as PR

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "libfullcheck.so")
OUTS = ("g", "p", "m", "v")
_lib = None


class Stats(ctypes.Structure):
    _fields_ = [("n_bad", ctypes.c_int64 * 4), ("first_bad", ctypes.c_int64 * 4),
                ("n_literal", ctypes.c_int64 * 4), ("worst", ctypes.c_double * 4),
                ("bf16_not_own", ctypes.c_int64), ("bf16_far", ctypes.c_int64),
                ("bf16_diff", ctypes.c_int64), ("first_bf16_bad", ctypes.c_int64)]

    def as_dict(self):
        d = {}
        for i, o in enumerate(OUTS):
            d[o] = {"bad": self.n_bad[i], "first_bad": self.first_bad[i],
                    "literal": self.n_literal[i], "worst": self.worst[i]}
        d["bf16"] = {"not_own": self.bf16_not_own, "far": self.bf16_far,
                     "diff_vs_oracle": self.bf16_diff, "first_bad": self.first_bf16_bad}
        return d


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.fullcheck_init.argtypes = [ctypes.POINTER(Stats)]
        L.fullcheck_init.restype = None
        L.fullcheck_block.argtypes = [i64, i64, vp, vp, vp, vp, i32, i64, i32, i64,
                                      f64, f64, f64, f64, f64, f64, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, ctypes.POINTER(Stats)]
        L.fullcheck_block.restype = None
        L.fullcheck_merge.argtypes = [ctypes.POINTER(Stats), ctypes.POINTER(Stats)]
        L.fullcheck_merge.restype = None
        L.fullcheck_rne.argtypes = [f64]
        L.fullcheck_rne.restype = ctypes.c_uint16
        _lib = L
    return _lib


def new_stats():
    s = Stats()
    lib().fullcheck_init(ctypes.byref(s))
    return s


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def check_block(base, p0, m0, v0, slices, slice_dtype, t, hp, ref, gpu_p, gpu_m, gpu_v,
                gpu_g=None, gpu_bf16=None, tol=PR.TOL):
    """Counts for one block of n elements (indices recorded as base + k).
    ``slices``: ``[N, n]`` raw slices (bf16 bits as uint16, or fp32); ``ref``:
    the oracle's float64 g, p, m, v; the GPU's fp32 results and, optionally,
    its stored gradient and bf16 copy (uint16 bits)."""
    bf16 = slice_dtype == "bf16"
    sl = np.ascontiguousarray(slices, dtype=np.uint16 if bf16 else np.float32)
    n_slices, n = sl.shape
    f32 = [np.ascontiguousarray(a, dtype=np.float32) for a in (p0, m0, v0, gpu_p, gpu_m, gpu_v)]
    r = [np.ascontiguousarray(ref[k], dtype=np.float64) for k in OUTS]
    g = None if gpu_g is None else np.ascontiguousarray(gpu_g, dtype=np.float32)
    b = None if gpu_bf16 is None else np.ascontiguousarray(gpu_bf16, dtype=np.uint16)
    for a in f32 + r + [x for x in (g, b) if x is not None]:
        assert a.shape == (n,)
    s = new_stats()
    lib().fullcheck_block(n, int(base), _p(f32[0]), _p(f32[1]), _p(f32[2]), _p(sl), int(bf16), n,
                          n_slices, int(t), float(hp["lr"]), float(hp["beta1"]),
                          float(hp["beta2"]), float(hp["eps"]), float(hp["weight_decay"]),
                          float(tol), _p(r[0]), _p(r[1]), _p(r[2]), _p(r[3]), _p(f32[3]),
                          _p(f32[4]), _p(f32[5]), _p(g), _p(b), ctypes.byref(s))
    return s


def rne(x):
    """The checker's bf16 rounding of each double in x (for its pin)."""
    f = lib().fullcheck_rne
    return np.array([f(float(v)) for v in np.asarray(x, dtype=np.float64).ravel()], dtype=np.uint16)


def merge(into, other):
    lib().fullcheck_merge(ctypes.byref(into), ctypes.byref(other))


def assert_ok(name, s, check_g=False, check_bf16=True):
    d = s.as_dict()
    for o in (("g",) if check_g else ()) + ("p", "m", "v"):
        assert d[o]["bad"] == 0, (f"{name} {o}: {d[o]['bad']} elements beyond tolerance, "
                                  f"first at {d[o]['first_bad']}")
    if check_bf16:
        assert d["bf16"]["not_own"] == 0 and d["bf16"]["far"] == 0, (
            f"{name} bf16: {d['bf16']['not_own']} not RNE of their own fp32, {d['bf16']['far']} "
            f"more than 1 ulp from RNE(oracle); first at {d['bf16']['first_bad']}")
    return d
