"""The quantizer's step Delta = fp32(m / qmax) is formed on the device without a division:
y = fp32(1/qmax), d0 = fp32(m y), r = m - qmax d0 (one fma, exact), Delta = fp32(d0 + r y)
(Markstein's correction step). This checks, in numpy with exact fp64 intermediates, that the
result equals IEEE fp32 division for qmax in {3, 7, 15} (symmetric INT3/INT4, zero-point
INT3/INT4) on every 4th fp32 significand (the full sweep of all 2^23 also passes; it takes a
few minutes). Every step scales exactly by powers of two in the range the device uses it for,
so one binade stands for all.
"""
import numpy as np
import pytest


def _corrected_quotient(m, b):
    bf = np.float32(b)
    y = np.float32(1) / bf
    d0 = m * y                                               # fp32 product, round to nearest
    r = m.astype(np.float64) - np.float64(b) * d0.astype(np.float64)   # exact in fp64
    assert np.array_equal(r.astype(np.float32).astype(np.float64), r)  # the fma's r is exact
    d = r * np.float64(y)                                    # exact: 24 x 24 bits
    # fp32(d0 + d) in one rounding: the nearest of d0 and its two neighbours, ties to even
    lo = np.nextafter(d0, np.float32(-np.inf))
    hi = np.nextafter(d0, np.float32(np.inf))
    cands = (lo, d0, hi)
    dist = [np.abs((c.astype(np.float64) - d0.astype(np.float64)) - d) for c in cands]
    pick = np.where(dist[0] < dist[1], 0, 1)
    pick = np.where(dist[2] < np.minimum(dist[0], dist[1]), 2, pick)
    out = np.choose(pick, cands)
    even = lambda x: (x.view(np.uint32) & 1) == 0
    out = np.where(dist[0] == dist[1], np.where(even(d0), d0, lo), out)
    out = np.where(dist[1] == dist[2], np.where(even(d0), d0, hi), out)
    return out, d0


@pytest.mark.parametrize("qmax", (3, 7, 15))
def test_corrected_product_equals_ieee_division(qmax):
    m = np.arange(0x3F800000, 0x40000000, 4, dtype=np.uint32).view(np.float32)
    q, d0 = _corrected_quotient(m, qmax)
    ref = m / np.float32(qmax)
    assert np.array_equal(q, ref)
    assert np.count_nonzero(d0 != ref) > m.size // 10   # the correction step does the work
