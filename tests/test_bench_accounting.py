"""The flop counts the benchmark divides by (bench.py) against an enumeration of the MFMAs the
Gram-form loss kernel issues: per grid point, 256-row tile of E' and 256-column tile lt, the K
loop runs min(8 (lt + 1), K / 32) steps of 32; in a full tile the last eight steps cover the
diagonal block of the lower-triangular operand, where the 32 x 32 x 16 products of column block c
(c = 2 j + wn for the wave's column half wn) at diagonal step d are issued only when d <= c (all
others multiply zeros). Runs on the CPU."""
import itertools

import pytest

import bench

MFMA_FLOPS = 2 * 32 * 32 * 16          # one v_mfma_f32_32x32x16_f16


def live(d, j, wn):
    """Whether block j of column half wn is issued at diagonal step d (d < 0: not a diagonal
    step)."""
    return d < 0 or d <= 2 * j or (d == 2 * j + 1 and wn == 1)


def enumerate_loss_flops(N, K, n_grid):
    t = -(-K // 256)
    tiles_n = -(-N // 256)
    mfmas = 0
    for lt in range(t):
        nk = min(8 * (lt + 1), K // 32)
        full = nk == 8 * (lt + 1)
        for step in range(nk):
            d = step - (nk - 8) if full and step >= nk - 8 else -1
            # 4 waves (wm, wn), 4 x 4 blocks (i, j), two k halves of 16
            for wm, wn, i, j, h in itertools.product(range(2), range(2), range(4), range(4),
                                                     range(2)):
                mfmas += live(d, j, wn)
    return mfmas * MFMA_FLOPS * tiles_n * n_grid


@pytest.mark.parametrize("N,K", [(4096, 4096), (256, 256), (300, 512), (4096, 11008),
                                 (1024, 8192), (512, 4224), (64, 160)])
def test_loss_executed_flops_match_the_kernel(N, K):
    assert bench.gram_loss_executed_flops(N, K, 20) == enumerate_loss_flops(N, K, 20)


def test_diagonal_rule_covers_exactly_the_triangle():
    """At diagonal step d (K rows 32 d .. 32 d + 31 of the block) column block c is issued iff
    some (k, l) in it has k <= l, i.e. iff d <= c: 36 of the 64 (step, column block) pairs."""
    issued = set()
    for d in range(8):
        for wn, j in itertools.product(range(2), range(4)):
            if live(d, j, wn):
                issued.add((d, 2 * j + wn))
    assert issued == {(d, c) for d in range(8) for c in range(8) if d <= c}
    assert len(issued) == 36


def test_method_flops():
    assert bench.gram_loss_flops(4096, 4096, 20) == 20 * 4096 * 4096 * 4096
    assert bench.gram_gemm_flops(65536, 4096) == 65536 * 4096 * 4096
    # the issued flops exceed the method's by the diagonal blocks only (0.8% at 4096 x 4096)
    ratio = bench.gram_loss_executed_flops(4096, 4096, 20) / bench.gram_loss_flops(4096, 4096, 20)
    assert 1.0 < ratio < 1.01
