"""The oracle's rank step in plain C (``oracle/rank_step.c``), loaded with ctypes.

Test infrastructure only (see ``oracle/__init__``).  Bit for bit the
arithmetic of ``oracle.step`` (the CPU tests check it), element by element in
compiled code, so that the parity tests can take the oracle over every
element of a rank shard of hundreds of millions of parameters.  ctypes
releases the GIL during a call, so calls on separate blocks run in parallel
on host threads.  The library is built by ``oracle/build.py`` (which
``__graft_entry__.build()`` runs); a missing library is an error.
"""

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboracle_step.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run python -m oracle.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_rank_step.argtypes = [vp, vp, vp, vp, i32, i64, i32, i64, i64,
                                       f64, f64, f64, f64, f64, vp, vp, vp, vp]
        L.oracle_rank_step.restype = ctypes.c_int
        L.oracle_rank_step_f64.argtypes = L.oracle_rank_step.argtypes
        L.oracle_rank_step_f64.restype = ctypes.c_int
        L.oracle_bf16_rne.argtypes = [vp, i64, vp]
        L.oracle_bf16_rne.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def rank_step(p, m, v, slices, slice_dtype, t, hp):
    """One rank step over every element of a block.

    ``p``, ``m``, ``v``: the state before the step (length n): fp32 arrays
    (the GPU's state, widened exactly) or float64 ones (the oracle's own
    trajectory).  ``slices``: ``[N, n]`` raw slices, bf16 bit patterns
    (uint16) when ``slice_dtype`` is "bf16", else fp32.  Returns a dict of
    float64 arrays g, p, m, v.
    """
    wide = np.asarray(p).dtype == np.float64
    dt = np.float64 if wide else np.float32
    p = np.ascontiguousarray(p, dtype=dt)
    m = np.ascontiguousarray(m, dtype=dt)
    v = np.ascontiguousarray(v, dtype=dt)
    bf16 = slice_dtype == "bf16"
    sl = np.ascontiguousarray(slices, dtype=np.uint16 if bf16 else np.float32)
    n_slices, n = sl.shape
    assert p.shape == m.shape == v.shape == (n,)
    out = {k: np.empty(n, dtype=np.float64) for k in ("g", "p", "m", "v")}
    f = lib().oracle_rank_step_f64 if wide else lib().oracle_rank_step
    rc = f(_ptr(p), _ptr(m), _ptr(v), _ptr(sl), int(bf16), n, n_slices, n, int(t), float(hp["lr"]),
           float(hp["beta1"]), float(hp["beta2"]), float(hp["eps"]), float(hp["weight_decay"]),
           _ptr(out["g"]), _ptr(out["p"]), _ptr(out["m"]), _ptr(out["v"]))
    if rc != 0:
        raise ValueError("oracle_rank_step: bad arguments")
    return out


def bf16_rne(x):
    """float64 values -> bf16 bit patterns (uint16), as oracle.step.bf16_rne."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_bf16_rne(_ptr(x), x.size, _ptr(out))
    return out
