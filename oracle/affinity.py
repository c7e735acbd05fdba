"""Expert affinity s = sqrt(softplus(l)), an fp32 value from an fp32 logit.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: mastering-deepseek-v4 "MoE + Expert-Parallel Overlap (Exp08)",
Implemented: top-k gating runs over Sqrt(Softplus(.)) affinities.

The pages name the function but not how to evaluate it.  Routing ranks
experts by it, so the evaluation has to (i) agree bit for bit with the GPU
when both start from the same fp32 logits and (ii) keep the order of the exact
function: sqrt(softplus(l)) is strictly increasing, so a larger logit must
never get a smaller affinity.  Both hold for this definition:

    s = fp32( sqrt( sp ) ),   sp = softplus(l) evaluated in fp64

by one fixed sequence of IEEE-754 fp64 operations (add, subtract, multiply,
divide, sqrt: each correctly rounded; rint, frexp, ldexp, abs, max: exact) with
no fused multiply-add, then a single rounding to fp32.  The fp64 value is
accurate to a few units in 2^-53, far finer than fp32's 2^-24 steps, so the
fp32 result is the correctly rounded affinity except within ~2^-50 of an
fp32 rounding boundary, and it is non-decreasing in l (an fp64 wobble could
only reverse the order where the exact function moves by less than that per
fp32 input step, i.e. for |l| below ~1e-8, and that range takes the branch
below that is monotone by construction).  numpy float64 ufuncs round each
operation on its own, so this module is such an implementation.

  l in fp64 (exact), a = |l|

  |l| < 2^-14:  sp = LN2 + (l/2 + (l*l)/8)        (Taylor series of softplus at
      0: ln2 + l/2 + l^2/8 - l^4/192 + ...; the dropped terms are < 2^-63 of sp.
      Every step is monotone in l, so the branch is too.)

  otherwise:    sp = max(l, 0) + log1p(exp(-a))   (the overflow-free form)

  exp(-a), 0 <= a <= 300  (Cody & Waite 1980, "Software Manual for the
      Elementary Functions": additive range reduction with ln2 split in two)
      n = rint(a * (1/ln2));  r = (n*LN2_HI - a) + n*LN2_LO,  |r| <~ ln2/2
      (LN2_HI = ln2 rounded to 40 significant bits, so n*LN2_HI is exact for
      n < 2^13; LN2_LO = fp64(ln2 - LN2_HI));  e^r by its degree-13 Taylor
      polynomial in Horner form (truncation < 2^-57 relative on |r| <= ln2/2);
      result = ldexp(p, -n).  For a > 300 the result is 0: there
      sqrt(softplus(l)) < e^-150, below half the smallest fp32 subnormal, so s
      rounds to 0 either way.

  log1p(u), 0 <= u <= 1  (Goldberg 1991, "What every computer scientist should
      know about floating-point arithmetic", Theorem 4: w = 1+u;
      log1p(u) = u if w == 1 else log(w) * u / (w - 1))
      log(w): w = m * 2^e with m in [sqrt(1/2), sqrt(2)); f = (m-1)/(m+1);
      log(m) = 2*atanh(f) = 2(f + f^3/3 + ... + f^21/21) (|f| <= 0.1716, next
      term < 2^-60 relative);  log(w) = e*LN2_HI + (log(m) + e*LN2_LO).

  s = fp32(sqrt(sp)): the fp64 square root is correctly rounded and rounding
      it again to fp32 equals rounding the exact square root of sp once
      (53 >= 2*24 + 2 bits: double rounding is innocuous for sqrt).

Pins (tests/test_oracle_affinity.py): non-decreasing over every fp32 logit in
[-210, 88] in order (exhaustive); equal to fp32(sqrt(logaddexp(0, l))) of fp64
libm on every fp32 logit in [-210, 88] except where that reference lies within
2^-44 (relative) of an fp32 rounding boundary; s(0) = fp32(sqrt(ln 2));
s(l) = fp32(sqrt(l)) once e^-l is below half an fp64 ulp of l; s = 0 for
l <= -210; the exp and log1p pieces against fp64 libm.
"""
from __future__ import annotations

import math

import numpy as np

f32 = np.float32
f64 = np.float64

INV_LN2 = float.fromhex("0x1.71547652b82fep+0")      # fp64(1/ln 2)
LN2_HI = float.fromhex("0x1.62e42fefa4000p-1")       # ln 2 to 40 significant bits
LN2_LO = float.fromhex("-0x1.8432a1b0e2634p-43")     # fp64(ln 2 - LN2_HI)
LN2 = LN2_HI + LN2_LO                                 # fp64(ln 2)
SQRT_HALF = math.sqrt(0.5)                            # fp64(sqrt(1/2))
SMALL = 2.0 ** -14                                    # Taylor branch below this |l|
EXP_CUTOFF = 300.0

# Taylor coefficients 1/i! for e^r, each the correctly rounded fp64 quotient
# (i! < 2^53 is exact).
EXP_C = [1.0 / math.factorial(i) for i in range(14)]
# Series coefficients 2/(2j+1) for 2*atanh(f).
LOG_C = [2.0 / (2 * j + 1) for j in range(11)]


def exp_neg(a):
    """fp64 e^{-a} for 0 <= a <= EXP_CUTOFF (see module header)."""
    a = np.asarray(a, dtype=f64)
    n = np.rint(a * INV_LN2)
    r = (n * LN2_HI - a) + n * LN2_LO
    p = np.full_like(r, EXP_C[13])
    for c in EXP_C[12::-1]:
        p = p * r + c
    return np.ldexp(p, (-n).astype(np.int32))


def log1p_unit(u):
    """fp64 log1p(u) for 0 <= u <= 1 (see module header)."""
    u = np.asarray(u, dtype=f64)
    w = u + 1.0
    m, e = np.frexp(w)
    low = m < SQRT_HALF
    m = np.where(low, m * 2.0, m)
    e = np.where(low, e - 1, e).astype(f64)
    f = (m - 1.0) / (m + 1.0)
    f2 = f * f
    q = np.full_like(f, LOG_C[10])
    for c in LOG_C[9::-1]:
        q = q * f2 + c
    logw = e * LN2_HI + (f * q + e * LN2_LO)
    with np.errstate(divide="ignore", invalid="ignore"):
        res = (logw * u) / (w - 1.0)
    return np.where(w == 1.0, u, res)


def softplus64(l):
    """fp64 softplus of fp32 logits (see module header)."""
    l = np.asarray(l, dtype=f32).astype(f64)
    a = np.abs(l)
    sp = np.empty_like(l)
    tiny = a < SMALL
    big = a > EXP_CUTOFF
    mid = ~(tiny | big)
    lt = l[tiny]
    sp[tiny] = LN2 + (lt * 0.5 + (lt * lt) * 0.125)
    lm = l[mid]
    sp[mid] = np.maximum(lm, 0.0) + log1p_unit(exp_neg(a[mid]))
    sp[big] = np.maximum(l[big], 0.0)
    return sp


def affinity(l):
    """fp32 s = sqrt(softplus(l)) from fp32 logits: one rounding of the fp64
    square root of the fp64 softplus."""
    scalar = np.ndim(l) == 0
    s = np.sqrt(softplus64(np.atleast_1d(l))).astype(f32)
    return s[0] if scalar else s
