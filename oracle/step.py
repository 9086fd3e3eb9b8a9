"""Oracle: the arithmetic of one rank's step, in float64 (NumPy).

Test infrastructure only (see ``oracle/__init__``).

The rank's work between the backward reduce-scatter and the next forward
all-gather, in the order the pages give it:

1. ``reduce_mean``   the N incoming gradient slices of this rank's shard are
   reduced to their mean.  FSDP chapter §18.3 and ZeRO state sharding post
   "ZeRO-2 方向：Gradient Sharding": backward ends in a reduce-scatter, each
   rank receiving only its reduced 1/N; FSDP chapter §18.6 and FSDP2 features
   doc "混合精度": the reduction runs in fp32 (reduce_dtype=float32).  Mean
   rather than sum: ZeRO state sharding post "Optimizer Step 的所有权" (every
   replica updates with the same averaged gradients) and its measured
   agreement of the sharded modes with plain DDP ("全模式性能结果与限制").
2. ``adamw``         the update runs on the local shard only, with no
   communication (FSDP chapter §18.21; ZeRO state sharding post "FSDP Sharded
   Optimizer"; FSDP2 features doc "工作原理", Update).  The optimizer is
   torch.optim.AdamW (FSDP chapter §18.43 recipe) with state exp_avg and
   exp_avg_sq (ZeRO state sharding post "三种 Model State").  The pages never
   print its equations; the reading taken is Adam (Kingma & Ba) with
   decoupled weight decay (Loshchilov & Hutter), the way torch.optim.AdamW
   applies it: decay by (1 - lr*wd) on the old parameter, both moments bias
   corrected, eps added after the square root of the corrected second moment.
3. ``bf16_rne``      the updated fp32 master is cast to bf16 for the next
   all-gather (FSDP chapter §18.6: parameters travel in bf16 while master
   weights stay fp32; §18.10: the low-precision cast runs before the
   all-gather).  Round to nearest, ties to even, from the IEEE definition.

Padding elements [valid, S) of every state and output buffer are exactly +0
(ZeRO state sharding post "FlatParameter 与 Padding").
"""

import numpy as np


# ---------------------------------------------------------------------------
# exact widening of the slice dtypes to float64


def widen_bf16_bits(u16):
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    u32 = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns widen to NaN
        return u32.view(np.float32).astype(np.float64)


def widen_f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# 1. reduce


def reduce_mean(slices_f64):
    """Mean over axis 0 of ``[N, n]`` float64 slices: (1/N) * sum_q x_q.

    The sum is taken in rank order 0..N-1 in float64, then divided by N once.
    """
    x = np.asarray(slices_f64, dtype=np.float64)
    n_slices = x.shape[0]
    acc = np.zeros(x.shape[1:], dtype=np.float64)
    for q in range(n_slices):
        acc = acc + x[q]
    return acc / n_slices


# ---------------------------------------------------------------------------
# 2. AdamW


def adamw(p, m, v, g, t, lr, beta1, beta2, eps, weight_decay):
    """One decoupled-weight-decay AdamW step in float64; returns (p', m', v').

        p1 = p * (1 - lr*wd)
        m' = beta1*m + (1 - beta1)*g
        v' = beta2*v + (1 - beta2)*g^2
        mhat = m' / (1 - beta1^t),  vhat = v' / (1 - beta2^t)
        p' = p1 - lr * mhat / (sqrt(vhat) + eps)

    ``t`` is the 1-based step count shared by every element.
    """
    assert t >= 1
    p = np.asarray(p, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    p1 = p * (1.0 - lr * weight_decay)
    m_new = beta1 * m + (1.0 - beta1) * g
    v_new = beta2 * v + (1.0 - beta2) * g * g
    mhat = m_new / (1.0 - beta1 ** t)
    vhat = v_new / (1.0 - beta2 ** t)
    p_new = p1 - lr * mhat / (np.sqrt(vhat) + eps)
    return p_new, m_new, v_new


# ---------------------------------------------------------------------------
# 3. bf16 round to nearest even

_BF16_FRAC_BITS = 7          # stored fraction bits
_EMIN = -126                 # smallest normal exponent (shared with fp32)
_EMAX = 127


def bf16_rne(x):
    """float64 values -> bf16 bit patterns (uint16), one correct RNE rounding.

    Written from the IEEE 754 definition of binary16-brain (1 sign, 8
    exponent, 7 fraction bits): the result is the representable value nearest
    to x, ties to the one with an even last fraction bit; magnitudes that
    round beyond the largest finite value give infinity; NaN gives the quiet
    NaN 0x7FC0 with x's sign; signed zeros keep their sign.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.zeros(flat.shape, dtype=np.uint16)
    sign = np.signbit(flat)
    a = np.abs(flat)
    nan = np.isnan(flat)
    inf = np.isinf(flat)
    fin = ~(nan | inf)

    # Exponent of the leading bit, and the spacing (ulp) of bf16 values there.
    af = np.where(fin & (a > 0), a, 1.0)
    _, e2 = np.frexp(af)             # af = f * 2**e2, 0.5 <= f < 1
    lead = e2 - 1                    # af in [2**lead, 2**(lead+1))
    lead = np.maximum(lead, _EMIN)   # below the normal range spacing is fixed
    ulp_exp = lead - _BF16_FRAC_BITS
    q = np.ldexp(af, -ulp_exp)       # exact: a power-of-two scaling
    qr = np.rint(q)                  # numpy rint = round half to even
    val = np.ldexp(qr, ulp_exp)      # exact bf16 value (or 2**(EMAX+1))
    val = np.where(fin & (a > 0), val, 0.0)
    over = fin & (val >= 2.0 ** (_EMAX + 1))
    val = np.where(over, 0.0, val)

    # Every finite bf16 value is exactly an fp32 value; its top 16 bits are it.
    bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[fin] = bits[fin]
    out[over] = 0x7F80
    out[inf] = 0x7F80
    out[nan] = 0x7FC0
    out = np.where(sign, out | np.uint16(0x8000), out).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f64(u16):
    return widen_bf16_bits(u16)


# ---------------------------------------------------------------------------
# the whole rank step on one shard buffer


def rank_step(p, m, v, slices_f64, valid, t, hp, grad_scale=None):
    """One rank step on one shard buffer of length S = len(p).

    ``slices_f64`` is ``[N, >=valid]`` (already widened); only the first
    ``valid`` columns are read.  ``hp`` holds lr, beta1, beta2, eps,
    weight_decay.  ``grad_scale`` (optional) multiplies the reduced gradient
    before the update: the clip coefficient of ``oracle.clip``.  Returns dict
    with g (the reduced gradient, unscaled), p, m, v (float64, length S) and
    bf16 (uint16 bits of RNE(p'), length S).  Positions >= valid are +0 in
    every output, whatever the inputs hold there.
    """
    S = len(p)
    g = np.zeros(S, dtype=np.float64)
    p_out = np.zeros(S, dtype=np.float64)
    m_out = np.zeros(S, dtype=np.float64)
    v_out = np.zeros(S, dtype=np.float64)
    if valid > 0:
        sl = np.asarray(slices_f64, dtype=np.float64)[:, :valid]
        g[:valid] = reduce_mean(sl)
        gu = g[:valid] if grad_scale is None else g[:valid] * grad_scale
        pv, mv, vv = adamw(p[:valid], m[:valid], v[:valid], gu, t,
                           hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                           hp["weight_decay"])
        p_out[:valid], m_out[:valid], v_out[:valid] = pv, mv, vv
    return {"g": g, "p": p_out, "m": m_out, "v": v_out, "bf16": bf16_rne(p_out)}
