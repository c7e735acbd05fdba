"""Expert affinity s = sqrt(softplus(l)) evaluated in fp32, one rounding per op.

Source: mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)",
Implemented: top-k gating runs over Sqrt(Softplus(.)) affinities.

The pages name the function but not how to evaluate it in fp32.  Routing has to
agree bit for bit with the GPU when both start from the same fp32 logits, so the
evaluation is fixed as a sequence of IEEE-754 fp32 operations (add, subtract,
multiply, divide, sqrt: each correctly rounded; rint, frexp, ldexp, abs:
exact), with no fused multiply-add.  Any implementation that performs the same
sequence gets the same bits.  numpy float32 ufuncs round each operation on its
own, so this module is such an implementation.

  softplus(l) = max(l, 0) + log1p(exp(-|l|))            (overflow-free form)

  exp(-a), a >= 0  (Cody & Waite 1980, "Software Manual for the Elementary
      Functions": additive range reduction with ln2 split in two parts)
      n = rint(a * (1/ln2));  r = (n*LN2_HI - a) + n*LN2_LO,  |r| <~ ln2/2
      e^r by its degree-7 Taylor polynomial in Horner form (truncation
      < 2^-27 relative on |r| <= ln2/2);  result = ldexp(p, -n).
      For a > 87 the result is flushed to 0 (e^-87 is the last value kept in
      the fp32 normal range).

  log1p(u), 0 <= u <= 1  (Goldberg 1991, "What every computer scientist should
      know about floating-point arithmetic", Theorem 4: w = 1+u;
      log1p(u) = u if w == 1 else log(w) * u / (w - 1))
      log(w): w = m * 2^e with m in [sqrt(1/2), sqrt(2)); f = (m-1)/(m+1);
      log(m) = 2*atanh(f) = 2(f + f^3/3 + ... + f^11/11) (|f| <= 0.1716, next
      term < 2^-33 relative);  log(w) = e*LN2_HI + (log(m) + e*LN2_LO).

Pins (tests/test_oracle_affinity.py): within 4 ulp of fp64
sqrt(logaddexp(0, l)) on a dense sweep of fp32 logits in [-87, 88] and on every
representable value in windows around 0 and elsewhere; monotone up to 3 ulp over
consecutive fp32 values; s(0) = fp32(sqrt(ln 2)); s(l) == fp32(sqrt(l)) once
exp(-l) falls below half an ulp of l.  The evaluation is not exactly monotone: it can
step back by up to 3 ulp between neighbouring inputs (pinned).
"""
from __future__ import annotations

import numpy as np

f32 = np.float32

# Constants as exact decimal expansions of fp32 values.
INV_LN2 = f32(1.44269502162933349609375)            # fp32(1/ln 2)
LN2_HI = f32(0.693359375)                           # 355/512: n*LN2_HI exact for n < 2^15
LN2_LO = f32(-0.000212194441701285541057586669922)   # fp32(ln2 - LN2_HI)
SQRT_HALF = f32(0.707106769084930419921875)         # fp32(sqrt(1/2))
EXP_CUTOFF = f32(87.0)
ONE = f32(1.0)
ZERO = f32(0.0)

# Taylor coefficients 1/i! for e^r, each a correctly rounded fp32 division.
_fact = [1, 1, 2, 6, 24, 120, 720, 5040]
EXP_C = [f32(1.0) / f32(_fact[i]) for i in range(8)]
# Series coefficients 2/(2j+1) for 2*atanh(f).
LOG_C = [f32(2.0) / f32(2 * j + 1) for j in range(6)]   # 2, 2/3, 2/5, 2/7, 2/9, 2/11


def _as_f32(x):
    return np.asarray(x, dtype=np.float32)


def exp_neg(a):
    """fp32 e^{-a} for a >= 0 (see module header)."""
    a = _as_f32(a)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint(a * INV_LN2)
        r = (n * LN2_HI - a) + n * LN2_LO
        p = EXP_C[7]
        for c in EXP_C[6::-1]:
            p = p * r + c
        res = np.ldexp(p, (-n).astype(np.int32)).astype(np.float32)
    return np.where(a > EXP_CUTOFF, ZERO, res).astype(np.float32)


def log1p_small(u):
    """fp32 log1p(u) for 0 <= u <= 1 (see module header)."""
    u = _as_f32(u)
    w = u + ONE
    m, e = np.frexp(w)
    m = m.astype(np.float32)
    low = m < SQRT_HALF
    m = np.where(low, m * f32(2.0), m).astype(np.float32)
    e = np.where(low, e - 1, e).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        f = (m - ONE) / (m + ONE)
        f2 = f * f
        q = LOG_C[5]
        for c in LOG_C[4::-1]:
            q = q * f2 + c
        logm = f * q
        logw = e * LN2_HI + (logm + e * LN2_LO)
        res = (logw * u) / (w - ONE)
    return np.where(w == ONE, u, res).astype(np.float32)


def softplus(l):
    """fp32 softplus(l) = max(l, 0) + log1p(exp(-|l|))."""
    l = _as_f32(l)
    pos = np.where(l > ZERO, l, ZERO).astype(np.float32)
    return pos + log1p_small(exp_neg(np.abs(l)))


def affinity(l):
    """fp32 s = sqrt(softplus(l)); the sqrt is correctly rounded."""
    return np.sqrt(softplus(l)).astype(np.float32)
