"""Oracle: fp8 all-gather copy of the updated shard with a per-tensor scale.

Test infrastructure only (see ``oracle/__init__``).

FSDP chapter §18.27 "FSDP x 量化训练 / 推理": lowering the all-gather dtype to
fp8 halves its bytes against bf16, but fp8's range is narrow, so each tensor
needs its own scale, carried with the quantised representation that is
gathered.  The page gives no recipe; the reading taken (the plainest dynamic
per-tensor scaling):

    amax_i  = max |p| over the whole tensor i (every rank's shard: the max of
              the ranks' local maxima; NaN propagates)
    scale_i = 448 / max(amax_i, 1e-12)                  (fp32)
    q       = RNE_e4m3(clamp(fp32(p * scale_i), -448, 448))

with OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits of bias 7, 3 fraction
bits, no infinities, largest finite 448, NaN = S.1111.111).  The product and
the scale are taken in fp32, the precision the device computes them in, so
that both sides decide the same integer code.  Padding codes are 0.
"""

import numpy as np

E4M3_MAX = 448.0
AMAX_FLOOR = 1e-12
_FRAC = 3
_EMIN = -6


def e4m3_rne(x):
    """float64 values (already within [-448, 448], or NaN) -> e4m3fn codes (uint8).

    Round to nearest, ties to even, from the definition: the result is the
    representable value nearest x; subnormals (below 2**-6) are spaced 2**-9.
    Values beyond the largest finite value saturate to +-448.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    sign = np.signbit(flat)
    a = np.abs(flat)
    nan = np.isnan(flat)
    af = np.where(nan | (a == 0), 1.0, np.minimum(a, E4M3_MAX))
    _, e2 = np.frexp(af)
    lead = np.maximum(e2 - 1, _EMIN)
    ulp_exp = lead - _FRAC
    q = np.rint(np.ldexp(af, -ulp_exp))            # exact scaling, then ties-to-even
    val = np.ldexp(q, ulp_exp)
    val = np.where(nan | (a == 0), 0.0, np.minimum(val, E4M3_MAX))
    # encode: exponent field and fraction
    _, ve = np.frexp(np.where(val > 0, val, 1.0))
    vlead = ve - 1
    normal = val >= 2.0 ** _EMIN
    frac_n = np.ldexp(val, -vlead) - 1.0                       # in [0, 1)
    code_n = ((vlead + 7) << 3) + np.rint(frac_n * 8).astype(np.int64)
    code_s = np.rint(np.ldexp(val, 9)).astype(np.int64)        # subnormal: val / 2**-9
    code = np.where(normal, code_n, code_s).astype(np.int64)
    code = np.where(nan, 0x7F, code)
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8).reshape(x.shape)


def e4m3_value(code):
    """e4m3fn codes -> float64 values (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = c & 0x7
    v = np.where(e == 0, np.ldexp(f.astype(np.float64), -9),
                 np.ldexp(1.0 + f / 8.0, e - 7))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return s * v


def amax(p):
    """max |p| (NaN propagates); 0 for an empty tensor."""
    p = np.asarray(p, dtype=np.float64)
    return float(np.max(np.abs(p))) if p.size else 0.0


def scale_of(amax_global):
    """fp32 scale from the global amax, computed in fp32."""
    a = np.float32(amax_global)
    floor = np.float32(AMAX_FLOOR)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.float32(E4M3_MAX) / (a if (a > floor or np.isnan(a)) else floor)


def quantize(p_f32, scale_f32):
    """fp8 codes of fp32 values with an fp32 scale: the product in fp32, then
    clamping and one RNE rounding."""
    p = np.asarray(p_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = (p * np.float32(scale_f32)).astype(np.float64)
    y = np.where(np.isnan(y), y, np.clip(y, -E4M3_MAX, E4M3_MAX))
    return e4m3_rne(y)
