"""Exact rational arithmetic used to pin the oracle on tiny inputs.

Independent of oracle/: every value is an exact Fraction and every fp32 rounding is done by
comparing the exact value with its neighbouring fp32 numbers.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np


def _f32_bits(x: np.float32) -> int:
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def rn32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 value, ties to the even significand."""
    if fr == 0:
        return np.float32(0.0)
    f = np.float32(float(fr))
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        key = (abs(Fraction(float(c)) - fr), _f32_bits(c) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def round_half_even(fr: Fraction) -> int:
    """Nearest integer to an exact rational, halves to the even integer."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def nearest_code(t: Fraction, qmin: int, qmax: int) -> int:
    """Exhaustive search over every code c in [qmin, qmax] for the one nearest to t
    (ties to the even code)."""
    best = None
    for c in range(qmin, qmax + 1):
        key = (abs(t - c), c % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def pow_rn32(x: float, a: float, digits: int = 45) -> np.float32:
    """fp32 rounding of x**a computed as exp(a ln x) with `digits` decimal digits."""
    if a == 0.0:
        return np.float32(1.0)
    with localcontext() as ctx:
        ctx.prec = digits
        v = (Decimal(a) * Decimal(x).ln()).exp()
    return rn32(Fraction(v))


def quantize_group_exact(w, s, qmin: int, qmax: int, ratio=None):
    """One group: ws = rn32(w s); with a clip ratio r, every ws is first moved into [-c, c],
    c = rn32(r max|ws|); Delta = rn32(max|ws| / qmax) of the (clipped) values; code = nearest
    code to rn32(ws / Delta). Returns (codes, Delta) with Delta an fp32 value."""
    ws = [Fraction(float(rn32(Fraction(float(wi)) * Fraction(float(si)))))
          for wi, si in zip(w, s)]
    m = max(abs(v) for v in ws)
    if ratio is not None:
        c = Fraction(float(rn32(Fraction(float(ratio)) * m)))
        ws = [min(max(v, -c), c) for v in ws]
        m = max(abs(v) for v in ws)
    if m == 0:
        return [0] * len(w), np.float32(0.0)
    delta = rn32(m / qmax)
    if delta == 0:
        return [0] * len(w), np.float32(0.0)
    codes = []
    for v in ws:
        t = rn32(v / Fraction(float(delta)))
        codes.append(nearest_code(Fraction(float(t)), qmin, qmax))
    return codes, delta


def group_error_exact(X, w, s, codes, delta):
    """sum_m ( sum_k X[m,k] (code_k Delta / s_k - w_k) )^2 over one group, exactly."""
    e = [Fraction(c) * Fraction(float(delta)) / Fraction(float(sk)) - Fraction(float(wk))
         for c, sk, wk in zip(codes, s, w)]
    tot = Fraction(0)
    for row in X:
        acc = sum(Fraction(float(x)) * ek for x, ek in zip(row, e))
        tot += acc * acc
    return tot


def loss_exact(X, W, codes, deltas, s, group: int) -> Fraction:
    """|| X E^T ||_F^2 / (M N) with E = q Delta / s - W, all exact."""
    M, K = X.shape
    N = W.shape[0]
    Xf = [[Fraction(float(X[m, k])) for k in range(K)] for m in range(M)]
    sf = [Fraction(float(v)) for v in s]
    E = []
    for n in range(N):
        row = []
        for k in range(K):
            d = Fraction(float(deltas[n][k // group]))
            row.append(Fraction(int(codes[n][k])) * d / sf[k] - Fraction(float(W[n, k])))
        E.append(row)
    tot = Fraction(0)
    for m in range(M):
        for n in range(N):
            y = sum(Xf[m][k] * E[n][k] for k in range(K))
            tot += y * y
    return tot / (M * N)


F16_MAX = Fraction(65504)
F16_OVERFLOW = Fraction(65520)   # 65504 + half an ulp of the top binade (2^15 / 2^10 / 2)


def rn16(fr: Fraction) -> np.float16:
    """Round an exact rational to the nearest fp16 value, ties to the even significand; IEEE 754
    overflow: a magnitude of at least 65520 (where rounding with an unbounded exponent would give
    2^16) becomes an infinity of that sign."""
    if fr == 0:
        return np.float16(0.0)
    if abs(fr) >= F16_OVERFLOW:
        return np.float16(np.inf) if fr > 0 else np.float16(-np.inf)
    f = np.float16(float(fr))
    with np.errstate(over="ignore"):
        cands = [f, np.nextafter(f, np.float16(np.inf)), np.nextafter(f, np.float16(-np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        bits = int(np.array(c, dtype=np.float16).view(np.uint16))
        key = (abs(Fraction(float(c)) - fr), bits & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float16(best[1])


def quantize_group_exact_zp(w, s, bits: int, ratio=None):
    """Zero-point quantization of one group: ws = rn32(w s) (clipped to +-rn32(r max|ws|) with a
    ratio); Delta = rn32(rn32(max - min) / (2^b - 1)); z = clamp(nearest integer to
    rn32(-min / Delta), 0, 2^b - 1); code = clamp(nearest integer to rn32(ws / Delta) + z, 0,
    2^b - 1). Returns (codes, Delta, z)."""
    qmax_u = 2 ** bits - 1
    ws = [Fraction(float(rn32(Fraction(float(wi)) * Fraction(float(si)))))
          for wi, si in zip(w, s)]
    if ratio is not None:
        c = Fraction(float(rn32(Fraction(float(ratio)) * max(abs(v) for v in ws))))
        ws = [min(max(v, -c), c) for v in ws]
    mx, mn = max(ws), min(ws)
    delta = rn32(Fraction(float(rn32(mx - mn))) / qmax_u)
    if delta == 0:
        return [0] * len(w), np.float32(0.0), 0
    d = Fraction(float(delta))
    z = min(max(round_half_even(Fraction(float(rn32(-mn / d)))), 0), qmax_u)
    codes = [min(max(round_half_even(Fraction(float(rn32(v / d)))) + z, 0), qmax_u) for v in ws]
    return codes, delta, z


def stats_sum_may_round(X, mantissa_bits: int) -> bool:
    """True when some column sum of |X| can round in fp64 for bf16 (7 fraction bits) or fp32 (23)
    values: every |x| of a column is a multiple of 2^(e - 127 - p), e the smallest exponent field
    of its non-zero values (1 for subnormals), so partial sums below 2^(53 + e - 127 - p) are
    exact. The column sum itself is taken with math.fsum (correctly rounded)."""
    import math
    X = np.asarray(X, dtype=np.float32)
    b = np.abs(X).view(np.uint32)
    f = (b >> 23).astype(np.int64)
    f = np.where(f == 0, 1, f)
    f = np.where(b == 0, 255, f)
    e = f.min(axis=0)
    for k in range(X.shape[1]):
        if e[k] == 255:
            continue
        S = math.fsum(np.abs(X[:, k]).astype(np.float64).tolist())
        if S >= math.ldexp(1.0, int(53 + e[k] - 127 - mantissa_bits)):
            return True
    return False
