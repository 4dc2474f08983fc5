"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test names the passage it follows. A plausible slip in the oracle -- a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding mode or step denominator -- fails
at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import exact_ref as ex

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _small_layer(seed, n, k, m, n_out=2, mult=8.0):
    g = np.random.default_rng(seed)
    W = (g.integers(-64, 65, size=(n, k)) / 256.0).astype(np.float16)
    X = g.integers(-16, 17, size=(m, k)) / 8.0
    X[:, g.choice(k, n_out, replace=False)] *= mult
    return W, X.astype(np.float16)


# --- P1: the equivalent transform ---------------------------------------------------------------
def test_p1_equivalent_transform_loss_vanishes_without_quantization():
    """"AWQ 量化方案..." section 二 (W X = (W/s)(X s)) and the AWQ notes' 方法 objective: with
    Q the identity, Q(W s)(s^-1 X) - W X = 0 for any positive s."""
    L = workloads.c1_layer()
    g = np.random.default_rng(11)
    s = np.exp(g.normal(0, 1.5, size=L.W.shape[1]))
    ref = (L.X.astype(np.float64) @ L.W.astype(np.float64).T)
    scale = float((ref * ref).mean())
    loss = oracle.output_loss(L.X, L.W, s, L.W.astype(np.float64) * s[None, :])
    assert loss / scale <= 1e-26
    # the opposite direction is a real error: the test can tell the two apart
    wrong = oracle.output_loss(L.X, L.W, s, L.W.astype(np.float64) / s[None, :])
    assert wrong / scale > 1e-2


# --- P2: alpha = 0 is plain round-to-nearest -----------------------------------------------------
def test_p2_alpha_zero_is_plain_rtn():
    """AWQ notes, 发现: RTN quantizes directly; at alpha = 0, s = s_X^0 = 1 exactly, so codes and
    loss reduce to per-group RTN. Reference RTN = torch's fp32 division and torch.round."""
    L = workloads.c1_layer()
    sx = oracle.act_stats(L.X)
    S = oracle.scale_table(sx, 20)
    assert np.all(S[0] == np.float32(1.0))
    q, delta = oracle.quantize(L.W, S[0], 4, 128)
    Wt = torch.from_numpy(L.W.astype(np.float32)).reshape(512, 4, 128)
    step = Wt.abs().amax(dim=2, keepdim=True) / 7.0
    q_rtn = torch.round(Wt / step).clamp(-8, 7).reshape(512, 512).to(torch.int8).numpy()
    assert np.array_equal(q, q_rtn)
    assert np.array_equal(delta, step.squeeze(2).numpy())
    Xd = torch.from_numpy(L.X.astype(np.float64))
    Wd = torch.from_numpy(L.W.astype(np.float64))
    Wq = torch.from_numpy(q_rtn.astype(np.float64)) * step.double().expand(-1, -1, 128).reshape(512, 512)
    rtn_loss = float(((Xd @ Wq.T - Xd @ Wd.T) ** 2).mean())
    res = oracle.search_layer(L.W, L.X, sx)
    assert res["losses"][0] == pytest.approx(rtn_loss, rel=1e-12)


# --- P3: the step formula ---------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 3])
def test_p3_step_reaches_qmax_and_never_qmin(bits):
    """Delta = max|ws| / (2^(b-1) - 1) ("AWQ 量化方案..." section 三, g_scale): the largest
    magnitude of each group maps to exactly +-qmax, and -2^(b-1) is never produced.
    (With the AWQ notes' 2^(b-1) denominator the maximum would map to 2^(b-1) and saturate.)"""
    L = workloads.c1_layer()
    S = oracle.scale_table(oracle.act_stats(L.X), 20)
    qmin, qmax = oracle.code_range(bits)
    for i in range(20):
        q, delta = oracle.quantize(L.W, S[i], bits, 128)
        ws = L.W.astype(np.float32) * S[i][None, :]
        qg = q.reshape(512, 4, 128)
        wsg = np.abs(ws.reshape(512, 4, 128))
        assert np.all(np.abs(qg).max(axis=2) == qmax)
        am = wsg.argmax(axis=2)
        assert np.all(np.abs(np.take_along_axis(qg, am[:, :, None], 2)) == qmax)
        assert not np.any(q == qmin)


# --- P4: rounding mode ------------------------------------------------------------------------
def test_p4_round_half_to_even_golden():
    rows = _golden_rows("round_half_even.txt")
    W = np.zeros((1, 128), dtype=np.float32)
    for j, (v, _) in enumerate(rows):
        W[0, j] = float(v)
    q, delta = oracle.quantize(W, np.ones(128, np.float32), 4, 128)
    assert delta[0, 0] == np.float32(1.0)
    assert [int(c) for c in q[0, :len(rows)]] == [int(c) for _, c in rows]


# --- P5: the pages' worked example -------------------------------------------------------------
def test_p5_worked_example_quantization_schemes():
    kv = dict(_golden_rows("worked_example_quant_schemes.txt"))
    r, w, a = float(kv["range_max"]), float(kv["weight"]), float(kv["activation"])
    W = np.zeros((1, 128), dtype=np.float32)
    W[0, 0], W[0, 1], W[0, 2] = r, w, -r
    s = np.ones(128, np.float32)
    q, delta = oracle.quantize(W, s, 4, 128)
    assert int(q[0, 1]) == int(kv["expected_code"])
    E = oracle.error_matrix(W, q, delta, s, 128)
    assert abs(E[0, 1]) == pytest.approx(float(kv["expected_weight_error"]), rel=1e-6)
    X = np.zeros((1, 128))
    X[0, 1] = a
    loss = oracle.output_loss(X, W, s, oracle.dequant_scaled(q, delta, 128))
    assert math.sqrt(loss) == pytest.approx(float(kv["expected_output_error"]), rel=1e-6)


# --- P6: a power-of-two factor on s changes no code -------------------------------------------
def test_p6_power_of_two_rescale_of_s_keeps_codes():
    """Normalising s (÷mean in the FlashAttention+AWQ page's AWQQuantizer, ÷max in section 三 of
    "AWQ 量化方案...") is a global factor; a power of two leaves every code bit-identical."""
    L = workloads.c1_layer()
    S = oracle.scale_table(oracle.act_stats(L.X), 20)
    for i in (0, 5, 12, 19):
        q1, d1 = oracle.quantize(L.W, S[i], 4, 128)
        q2, d2 = oracle.quantize(L.W, S[i] * np.float32(4.0), 4, 128)
        assert np.array_equal(q1, q2)
        assert np.array_equal(d2, d1 * np.float32(4.0))


# --- P7: the error-ratio argument --------------------------------------------------------------
def test_p7_scaling_one_channel_by_two_halves_its_error():
    """AWQ notes, 方法: rounding error is uniform on [0, 0.5] steps; scaling one weight by s > 1
    barely moves the group maximum, so its error in original units shrinks by Delta'/Delta * 1/s.
    With s = 2 on a non-maximal channel the step is unchanged and the mean error halves."""
    g = np.random.default_rng(7)
    G = 100_000
    W = g.standard_normal((G, 128)).astype(np.float32)
    m = np.abs(W).max(axis=1)
    cand = np.abs(W) < (m[:, None] / 2)
    k = np.argmax(np.where(cand, g.random((G, 128)), -1.0), axis=1)   # a random admissible channel
    ones = np.ones(128, np.float32)
    q1, d1 = oracle.quantize(W, ones, 4, 128)
    err1 = np.abs(oracle.error_matrix(W, q1, d1, ones, 128)[np.arange(G), k])
    err2 = np.empty(G)
    d2 = np.empty(G, np.float32)
    # one row at a time would be slow; group rows by their chosen channel
    for kk in range(128):
        rows = np.flatnonzero(k == kk)
        if rows.size == 0:
            continue
        s = ones.copy()
        s[kk] = 2.0
        q, d = oracle.quantize(W[rows], s, 4, 128)
        err2[rows] = np.abs(oracle.error_matrix(W[rows], q, d, s, 128)[:, kk])
        d2[rows] = d[:, 0]
    assert np.array_equal(d2, d1[:, 0])
    ratio = err2.mean() / err1.mean()
    assert abs(ratio - 0.5) < 0.01


# --- P8: brute force on tiny layers ------------------------------------------------------------
@pytest.mark.parametrize("seed,n,k,m,bits", [(1, 2, 128, 3, 4), (2, 3, 256, 5, 4),
                                             (3, 2, 256, 4, 3)])
def test_p8_brute_force_tiny_layer(seed, n, k, m, bits):
    """Every code is the nearest of all 2^b codes to the fp32 quotient (ties to even), every loss
    is the exact rational ||X E^T||^2/(MN), and alpha* is the exhaustive argmin."""
    W, X = _small_layer(seed, n, k, m)
    n_grid = 6
    sx = oracle.act_stats(X)
    for kk in range(k):
        exact = Fraction(sum(abs(Fraction(float(v))) for v in X[:, kk])) / m
        assert sx[kk] == ex.rn32(exact)
    res = oracle.search_layer(W, X, sx, bits=bits, group=128, n_grid=n_grid)
    qmin, qmax = oracle.code_range(bits)
    exact_losses = []
    for i in range(n_grid):
        s = res["scales"][i]
        q, delta = oracle.quantize(W, s, bits, 128)
        codes, deltas = [], []
        for r in range(n):
            row_c, row_d = [], []
            for g0 in range(0, k, 128):
                c, d = ex.quantize_group_exact(W[r, g0:g0 + 128], s[g0:g0 + 128], qmin, qmax)
                row_c += c
                row_d.append(d)
            codes.append(row_c)
            deltas.append(row_d)
        assert np.array_equal(q, np.array(codes, dtype=np.int8))
        assert np.array_equal(delta, np.array(deltas, dtype=np.float32))
        le = ex.loss_exact(X, W, codes, deltas, s, 128)
        exact_losses.append(le)
        assert res["losses"][i] == pytest.approx(float(le), rel=1e-12)
    best = min(range(n_grid), key=lambda i: (exact_losses[i], i))
    assert res["best"] == best


# --- P9: direct and Gram forms -----------------------------------------------------------------
def test_p9_direct_and_gram_forms_agree():
    """The GPTQ section of "量化方案详解" writes the layer objective as (W - Wq)^T H (W - Wq)
    with H = X^T X; the same identity gives ||X E^T||^2 = sum_n E_n H E_n^T."""
    L = workloads.c1_layer()
    sx = oracle.act_stats(L.X)
    d = oracle.search_layer(L.W, L.X, sx, form="direct")
    g = oracle.search_layer(L.W, L.X, sx, form="gram")
    np.testing.assert_allclose(g["losses"], d["losses"], rtol=1e-12)
    Ls = workloads.c2_like_layer(n=192, k=384, m=1500, config=2)
    sx = oracle.act_stats(Ls.X)
    d = oracle.search_layer(Ls.W, Ls.X, sx, form="direct")
    g = oracle.search_layer(Ls.W, Ls.X, sx, form="gram")
    np.testing.assert_allclose(g["losses"], d["losses"], rtol=1e-12)
    assert d["best"] == g["best"]


# --- P10: activation statistics -----------------------------------------------------------------
def test_p10_stats_constant_column_and_order_independence():
    g = np.random.default_rng(5)
    X = (g.standard_normal((3000, 256)) * np.exp(g.normal(0, 2, 256))).astype(np.float16)
    X[:, 7] = np.float16(-1.375)
    X[:, 9] = np.float16(6.1e-5)           # fp16 subnormal magnitudes still sum exactly
    sx = oracle.act_stats(X)
    assert sx[7] == np.float32(1.375)
    assert sx[9] == np.float32(float(np.float16(6.1e-5)))
    perm = g.permutation(3000)
    assert np.array_equal(oracle.act_stats(X[perm]), sx)
    assert np.array_equal(oracle.act_stats(X, chunk_rows=7), sx)
    for kk in (0, 100, 255):
        exact = Fraction(math.fsum(abs(float(v)) for v in X[:, kk])) / 3000
        assert sx[kk] == ex.rn32(exact)


# --- P11: packing ------------------------------------------------------------------------------
def test_p11_pack_golden_and_roundtrip():
    rows = _golden_rows("pack_nibbles.txt")
    q = np.array([[int(v) for v in r[:8]] for r in rows], dtype=np.int8)
    words = oracle.pack_int4(q)
    assert [int(w[0]) for w in words] == [int(r[8], 16) for r in rows]
    g = np.random.default_rng(3)
    q = g.integers(-8, 8, size=(37, 256), dtype=np.int8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q)), q)


# --- P12: W4A16 ---------------------------------------------------------------------------------
def test_p12_w4a16_integer_case_and_exact_rationals():
    """"AWQ 量化方案..." section 三, QuantLinear.forward: unit steps and s make the product an
    integer matmul; general fp16 steps and s checked against exact rationals."""
    g = np.random.default_rng(9)
    q = g.integers(-8, 8, size=(24, 256), dtype=np.int8)
    A = g.integers(-3, 4, size=(5, 256)).astype(np.float16)
    qw = oracle.pack_int4(q)
    y = oracle.w4a16(A, qw, np.ones((24, 2), np.float16), np.ones(256, np.float16), 128)
    assert np.array_equal(y, (A.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64))
    sc = (0.01 * np.abs(g.standard_normal((24, 2))) + 1e-3).astype(np.float16)
    s = (1 + np.abs(g.standard_normal(256))).astype(np.float16)
    A = g.standard_normal((3, 256)).astype(np.float16)
    y = oracle.w4a16(A, qw, sc, s, 128)
    for mm in range(3):
        for nn in (0, 5, 23):
            e = sum(Fraction(float(A[mm, kk])) / Fraction(float(s[kk])) * int(q[nn, kk]) *
                    Fraction(float(sc[nn, kk // 128])) for kk in range(256))
            assert y[mm, nn] == pytest.approx(float(e), rel=1e-13, abs=1e-300)


# --- grid and scale table ----------------------------------------------------------------------
def test_scale_table_matches_high_precision_power():
    """s_i = fp32(max(s_X, 1e-5)^alpha_i) (AWQ notes 方法: s = s_X^alpha, alpha in [0, 1]),
    checked against a 45-digit exp(alpha ln x) correctly rounded to fp32; ends exact."""
    L = workloads.c1_layer()
    sx = oracle.act_stats(L.X)
    S = oracle.scale_table(sx, 20)
    base = np.maximum(sx, np.float32(1e-5))
    assert np.array_equal(S[-1], base)
    assert np.all(S[0] == 1.0)
    alphas = oracle.alpha_grid(20)
    assert alphas[0] == 0.0 and alphas[-1] == 1.0 and alphas[5] == 5 / 19
    for i in range(1, 19):
        for kk in range(0, 512, 7):
            assert S[i, kk] == ex.pow_rn32(float(base[kk]), alphas[i]), (i, kk)


def test_floor_applies_to_dead_channels():
    sx = np.array([0.0, 1e-7, 2.0], np.float32)
    S = oracle.scale_table(sx, 3)
    f = np.float32(1e-5)
    assert S[2, 0] == f and S[2, 1] == f and S[2, 2] == np.float32(2.0)
    assert S[1, 0] == np.float32(math.sqrt(float(f)))


def test_argmin_takes_lowest_index_on_ties():
    assert oracle.argmin_lowest([3.0, 1.0, 1.0, 2.0]) == 1
    assert oracle.argmin_lowest([1.0, 1.0]) == 0


def test_all_zero_group_has_zero_step_and_codes():
    W = np.zeros((2, 256), np.float32)
    W[1, 200] = 0.5
    q, d = oracle.quantize(W, np.ones(256, np.float32), 4, 128)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0 and d[1, 1] == np.float32(0.5 / 7)
    assert np.count_nonzero(q) == 1 and q[1, 200] == 7


def test_search_improves_on_rtn_for_outlier_layer():
    """AWQ notes, 方法: protecting the salient channels lowers the output error, so on a layer
    with outlier activation channels some alpha > 0 beats alpha = 0 (RTN)."""
    L = workloads.c1_layer()
    res = oracle.search_layer(L.W, L.X, oracle.act_stats(L.X))
    assert res["best"] > 0
    assert res["losses"][res["best"]] < 0.6 * res["losses"][0]


def test_nonfinite_inputs_are_rejected():
    W = np.ones((1, 128), np.float32)
    W[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize(W, np.ones(128, np.float32))
    with pytest.raises(ValueError):
        oracle.act_stats(np.array([[np.inf, 1.0]]))


# --- P13: clipping (R17) ---------------------------------------------------------------------
def _outlier_layer(seed, n, k, m):
    """Groups with a few large weights of either sign among small ones, so that clipping
    changes codes in both directions."""
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((n, k))).astype(np.float32)
    for r in range(n):
        for g0 in range(0, k, 128):
            idx = g.choice(128, 2, replace=False) + g0
            W[r, idx] = np.float32(0.3) * np.sign(g.standard_normal(2)).astype(np.float32)
    X = g.standard_normal((m, k)).astype(np.float32)
    s = np.exp(0.3 * g.standard_normal(k)).astype(np.float32)
    return W, X, s


def test_p13_ratio_one_is_the_unclipped_quantizer():
    W, X, s = _outlier_layer(60, 7, 384, 5)
    q0, d0 = oracle.quantize(W, s, 4, 128)
    q1, d1 = oracle.quantize(W, s, 4, 128, clip=np.ones((7, 3), np.float32))
    assert np.array_equal(q0, q1) and np.array_equal(d0, d1)


def test_p13_group_errors_add_up_to_the_output_loss():
    """For a single-group layer the group errors of all rows add up to M N L of the literal
    objective (output_loss); for several groups the direct and Gram evaluations agree."""
    W, X, s = _outlier_layer(61, 9, 128, 40)
    q, d = oracle.quantize(W, s, 4, 128)
    err = oracle.group_errors(oracle.error_matrix(W, q, d, s), 128, X=X)
    L = oracle.output_loss(X, W, s, oracle.dequant_scaled(q, d))
    assert err.sum() == pytest.approx(L * X.shape[0] * W.shape[0], rel=1e-12)
    W2, X2, s2 = _outlier_layer(62, 5, 512, 30)
    q2, d2 = oracle.quantize(W2, s2, 4, 128)
    E2 = oracle.error_matrix(W2, q2, d2, s2)
    np.testing.assert_allclose(oracle.group_errors(E2, 128, X=X2),
                               oracle.group_errors(E2, 128, H=oracle.gram(X2)), rtol=1e-11)


@pytest.mark.parametrize("bits", [4, 3])
def test_p13_clip_search_brute_force_exact(bits):
    """Every clipped code is the nearest code to the fp32 quotient of the clipped value, every
    group error equals the exact rational, and each (row, group) gets the exhaustive argmin."""
    W, X, s = _outlier_layer(63 + bits, 3, 256, 6)
    n_clip, clip_min = 6, 0.4
    res = oracle.clip_search(W, X, s, bits=bits, n_clip=n_clip, clip_min=clip_min)
    ratios = oracle.clip_grid(n_clip, clip_min)
    qmin, qmax = oracle.code_range(bits)
    for n in range(3):
        for g in range(2):
            sl = slice(128 * g, 128 * (g + 1))
            errs = []
            for j, r in enumerate(ratios):
                codes, delta = ex.quantize_group_exact(W[n, sl], s[sl], qmin, qmax, ratio=r)
                q, d = oracle.quantize(W, s, bits, 128, clip=np.full((3, 2), r, np.float32))
                assert list(q[n, sl]) == codes and d[n, g] == delta, (n, g, j)
                e = ex.group_error_exact(X[:, sl], W[n, sl], s[sl], codes, delta)
                errs.append(e)
                assert res["err"][j, n, g] == pytest.approx(float(e), rel=1e-12)
            best = min(range(n_clip), key=lambda j: (errs[j], j))
            assert res["best"][n, g] == best
            assert res["ratio"][n, g] == ratios[best]


def test_p13_clipping_helps_an_outlier_group():
    """One weight of 1 among 127 weights of 0.06, unit activations on every channel (X = I):
    unclipped, the step is 1/7 and every small weight rounds to 0 (error 127 * 0.06^2); half-way
    clipping (r = 0.5) costs 0.5^2 on the outlier but represents the small weights (code 1,
    step 1/14), so the search must leave r = 1."""
    W = np.full((1, 128), 0.06, np.float32)
    W[0, 0] = 1.0
    X = np.eye(128, dtype=np.float32)
    s = np.ones(128, np.float32)
    res = oracle.clip_search(W, X, s, n_clip=11, clip_min=0.5)
    w_small = float(np.float32(0.06))
    assert res["err"][0, 0, 0] == pytest.approx(127 * w_small ** 2, rel=1e-6)
    r05 = 0.25 + 127 * (w_small - 1 / 14) ** 2
    assert res["err"][10, 0, 0] == pytest.approx(r05, rel=1e-5)
    assert res["best"][0, 0] > 0 and res["err"][res["best"][0, 0], 0, 0] <= r05


def test_p13_ties_keep_the_lowest_ratio_index():
    """A zero weight group, or a group whose channels never activate, has error 0 at every
    ratio: the first grid point (r = 1, no clipping) is kept (R10)."""
    W, X, s = _outlier_layer(67, 4, 256, 8)
    W[1, :128] = 0
    X[:, 128:] = 0
    res = oracle.clip_search(W, X, s, n_clip=5, clip_min=0.5)
    assert res["best"][1, 0] == 0 and res["ratio"][1, 0] == np.float32(1.0)
    assert (res["best"][:, 1] == 0).all() and (res["err"][:, :, 1] == 0).all()



# --- P14: shared scale and folding (R18) -----------------------------------------------------
def test_p14_shared_loss_is_the_row_weighted_mean_of_the_layer_losses():
    """One s for several weights: at every grid point the loss over the concatenated rows is the
    row-count-weighted mean of each weight's own loss (search_layer) at that s."""
    g = np.random.default_rng(70)
    X = (g.standard_normal((120, 256)) * np.exp(g.standard_normal(256))).astype(np.float32)
    Ws = [(0.02 * g.standard_normal((n, 256))).astype(np.float32) for n in (40, 16, 72)]
    sx = oracle.act_stats(X)
    sh = oracle.search_shared(Ws, X, sx, n_grid=7)
    per = [oracle.search_layer(W, X, sx, n_grid=7)["losses"] for W in Ws]
    want = sum(n * L for n, L in zip((40, 16, 72), per)) / 128
    np.testing.assert_allclose(sh["losses"], want, rtol=1e-12)
    assert sh["best"] == int(np.argmin(want))


def test_p14_fold_is_the_correctly_rounded_quotient():
    """fp16 and fp32 parameters: each folded value is the fp16 (fp32) value nearest to the fp32
    quotient, both axes."""
    g = np.random.default_rng(71)
    s = np.exp(g.standard_normal(24)).astype(np.float32)
    for dt, rn in ((np.float16, ex.rn16), (np.float32, lambda fr: np.float32(ex.rn32(fr)))):
        gamma = (1 + 0.1 * g.standard_normal((1, 24))).astype(dt)
        f1 = oracle.fold_scale(gamma, s, axis=1)
        Wp = (0.05 * g.standard_normal((24, 5))).astype(dt)
        f0 = oracle.fold_scale(Wp, s, axis=0)
        for k in range(24):
            q = ex.rn32(Fraction(float(gamma[0, k])) / Fraction(float(s[k])))
            assert f1[0, k] == rn(Fraction(float(q)))
            for c in range(5):
                q = ex.rn32(Fraction(float(Wp[k, c])) / Fraction(float(s[k])))
                assert f0[k, c] == rn(Fraction(float(q)))


def test_p14_folding_then_the_scaled_layer_reproduces_the_layer():
    """With s a power of two per channel, folding s^-1 into a norm weight and multiplying the
    layer's weight by s changes nothing at all: (x gamma / s) (W s)^T == (x gamma) W^T exactly;
    and W4A16 on the folded input without the division equals W4A16 with it."""
    g = np.random.default_rng(72)
    K = 256
    s = np.exp2(g.integers(-3, 4, K)).astype(np.float32)
    gamma = (1 + 0.1 * g.standard_normal((1, K))).astype(np.float32)
    x = g.standard_normal((6, K)).astype(np.float32)
    W = (0.02 * g.standard_normal((10, K))).astype(np.float32)
    gf = oracle.fold_scale(gamma, s, axis=1)
    lhs = (x.astype(np.float64) * gf.astype(np.float64)) @ (W.astype(np.float64) * s).T
    rhs = (x.astype(np.float64) * gamma.astype(np.float64)) @ W.astype(np.float64).T
    assert np.array_equal(lhs, rhs)
    p = oracle.pack_layer(W, s)
    A = (x * gamma).astype(np.float16)
    Af = (A.astype(np.float32) / s[None, :]).astype(np.float16)   # exact: s is 2^k
    np.testing.assert_array_equal(oracle.w4a16(Af, p["qweight"], p["scales16"], None),
                                  oracle.w4a16(A, p["qweight"], p["scales16"], p["s16"]))


def test_p14_w4a16_without_s_exact_on_a_tiny_case():
    """W4A16 with the division folded away: Y = A (q step)^T, checked with exact rationals."""
    g = np.random.default_rng(73)
    q = g.integers(-8, 8, size=(3, 128)).astype(np.int8)
    step = (0.01 * (1 + g.random((3, 1)))).astype(np.float16)
    A = g.standard_normal((2, 128)).astype(np.float16)
    Y = oracle.w4a16(A, oracle.pack_int4(q), step, None)
    for m in range(2):
        for n in range(3):
            want = sum(Fraction(float(A[m, k])) * int(q[n, k]) * Fraction(float(step[n, 0]))
                       for k in range(128))
            assert Y[m, n] == pytest.approx(float(want), rel=1e-13, abs=1e-15)



# --- P15: zero-point quantization (R19) --------------------------------------------------------
def test_p15_worked_example_of_the_quantization_schemes_page():
    """"量化方案详解", section AWQ: weights spanning [-3.2, 3.2] on 16 levels have the step
    0.427; w = 0.21 is quantized to 0 (error 0.21), an output error of 21 at activation 100."""
    W = np.zeros((1, 128), np.float32)
    W[0, :3] = [-3.2, 3.2, 0.21]
    q, d, z = oracle.quantize_zp(W, np.ones(128, np.float32), bits=4)
    assert round(float(d[0, 0]), 3) == 0.427
    level = (int(q[0, 2]) - int(z[0, 0])) * float(d[0, 0])
    assert level == 0.0
    assert abs(float(np.float32(0.21)) - level) == pytest.approx(0.21, abs=1e-7)
    assert 100 * abs(float(np.float32(0.21)) - level) == pytest.approx(21, abs=1e-5)


@pytest.mark.parametrize("bits,group", [(4, 128), (3, 64), (4, 64)])
def test_p15_zero_point_brute_force_exact(bits, group):
    """Codes, steps and zero points against exact rationals (with and without clipping), and
    the search's losses against the exact rational objective with (q - z) Delta."""
    W, X = _small_layer(90 + bits + group, 3, 256, 5)
    W[1, :group] = np.abs(W[1, :group])          # a group with min >= 0: z clamps to 0
    s = np.exp(0.3 * np.random.default_rng(91).standard_normal(256)).astype(np.float32)
    for ratio in (None, np.float32(0.7)):
        clip = None if ratio is None else np.full((3, 256 // group), ratio, np.float32)
        q, d, z = oracle.quantize_zp(W, s, bits, group, clip=clip)
        for n in range(3):
            for g in range(256 // group):
                sl = slice(g * group, (g + 1) * group)
                c, dd, zz = ex.quantize_group_exact_zp(W[n, sl], s[sl], bits, ratio=ratio)
                assert list(q[n, sl]) == c and d[n, g] == dd and z[n, g] == zz, (n, g, ratio)
    assert z[1, 0] == 0
    sx = oracle.act_stats(X)
    res = oracle.search_layer(W, X, sx, bits=bits, group=group, n_grid=4, zero_point=True)
    for i in range(4):
        q, d, z = oracle.quantize_zp(W, res["scales"][i], bits, group)
        centred = q.astype(np.int64) - np.repeat(z.astype(np.int64), group, axis=1)
        le = ex.loss_exact(X, W, centred, d, res["scales"][i], group)
        assert res["losses"][i] == pytest.approx(float(le), rel=1e-12)


def test_p15_zero_point_pack_and_w4a16():
    """Unsigned nibbles round-trip; W4A16 with zero points against exact rationals."""
    g = np.random.default_rng(92)
    q = g.integers(0, 16, size=(3, 256)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_uint4(oracle.pack_int4(q)), q)
    z = g.integers(0, 16, size=(3, 2)).astype(np.uint8)
    step = (0.01 * (1 + g.random((3, 2)))).astype(np.float16)
    s16 = (1 + g.random(256)).astype(np.float16)
    A = g.standard_normal((2, 256)).astype(np.float16)
    Y = oracle.w4a16(A, oracle.pack_int4(q), step, s16, zeros=z)
    for m in range(2):
        for n in range(3):
            want = sum(Fraction(float(A[m, k])) / Fraction(float(s16[k])) *
                       (int(q[n, k]) - int(z[n, k // 128])) * Fraction(float(step[n, k // 128]))
                       for k in range(256))
            assert Y[m, n] == pytest.approx(float(want), rel=1e-12, abs=1e-14)


# --- P16: group 64 -----------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [4, 3])
def test_p16_group64_brute_force_exact(bits):
    W, X = _small_layer(95 + bits, 3, 256, 4)
    s = np.exp(0.3 * np.random.default_rng(96).standard_normal(256)).astype(np.float32)
    qmin, qmax = oracle.code_range(bits)
    q, d = oracle.quantize(W, s, bits, 64)
    for n in range(3):
        for g in range(4):
            sl = slice(64 * g, 64 * (g + 1))
            c, dd = ex.quantize_group_exact(W[n, sl], s[sl], qmin, qmax)
            assert list(q[n, sl]) == c and d[n, g] == dd


def test_p16_group64_equals_group128_when_both_halves_hold_the_maximum():
    """If both 64-channel halves of every 128-channel group reach the group's max |w s|, the
    steps coincide and group 64 gives the codes of group 128."""
    g = np.random.default_rng(97)
    W = (0.02 * g.standard_normal((5, 512))).astype(np.float32)
    s = np.ones(512, np.float32)
    for r in range(5):
        for g0 in range(0, 512, 128):
            m = np.abs(W[r, g0:g0 + 128]).max()
            W[r, g0] = m
            W[r, g0 + 64] = -m
    q64, d64 = oracle.quantize(W, s, 4, 64)
    q128, d128 = oracle.quantize(W, s, 4, 128)
    assert np.array_equal(q64, q128)
    assert np.array_equal(d64, np.repeat(d128, 2, axis=1))


# --- fp16 storage of steps and s, and the checks' own metrics -----------------------------------
def _f16_boundary_values():
    """Exact rationals at the places where an fp16 rounding goes wrong most easily."""
    two = Fraction(2)
    return [
        Fraction(1) + two ** -11,                 # tie between 1 and 1 + 2^-10: to even (1)
        Fraction(1) + 3 * two ** -11,             # tie: to even (1 + 2^-9)
        Fraction(1) + two ** -11 + two ** -20,    # just above the tie: up
        two ** -14,                               # smallest normal
        two ** -14 - two ** -25,                  # tie between the largest subnormal and 2^-14
        two ** -14 - 3 * two ** -25,              # tie between two subnormals: to even
        two ** -25,                               # half the smallest subnormal: to 0 (even)
        3 * two ** -26,                           # above that half: the smallest subnormal
        Fraction(65504),                          # largest finite
        Fraction(65519),                          # rounds down to 65504
        Fraction(65520),                          # the overflow threshold: Inf
        Fraction(3, 10), Fraction(1, 3), Fraction(7, 5) * two ** -20,
    ]


def test_pack_stores_steps_and_s_as_correctly_rounded_fp16():
    """"AWQ 量化方案..." section 三 stores per-group FP16 scales and the per-channel scale: the
    oracle's fp16 steps and s must be the correctly rounded fp16 of the fp32 values (ties to
    even, subnormals, overflow to Inf), checked here against exact rationals at every boundary
    case rather than against numpy's own cast."""
    vals = _f16_boundary_values()
    # s16: pack_layer rounds the given fp32 s; each value is first made an fp32 number
    s32 = np.array([np.float32(float(v)) for v in vals], dtype=np.float32)
    # the boundary cases must survive fp32 exactly for the pin to mean what it says
    for v, f in zip(vals[:11], s32[:11]):
        assert Fraction(float(f)) == v
    K = 128 * ((len(vals) + 127) // 128)
    s = np.ones(K, np.float32)
    s[:len(vals)] = s32
    W = np.zeros((len(vals), K), np.float32)
    # steps: row r has one group whose max |w s| is 7 * target, so Delta = fp32(7 t / 7) = t
    for r, f in enumerate(s32):
        W[r, len(vals)] = np.float32(7.0) * f          # channel with s = 1
    with np.errstate(over="ignore"):
        o = oracle.pack_layer(W, s, bits=4, group=128)
    for j, f in enumerate(s32):
        want = ex.rn16(Fraction(float(f)))
        got = o["s16"][j]
        assert (np.isinf(want) and np.isinf(got)) or got == want, (float(f), got, want)
        d = o["delta"][j, len(vals) // 128]
        if j < 11:          # 7 t is exact in fp32 there, so Delta = t is the boundary value
            assert d == f
        want_d = ex.rn16(Fraction(float(d)))
        got_d = o["scales16"][j, len(vals) // 128]
        assert (np.isinf(want_d) and np.isinf(got_d)) or got_d == want_d, (float(f), got_d)
    # spot values the exact rounding must give
    assert ex.rn16(vals[0]) == np.float16(1.0)
    assert ex.rn16(vals[1]) == np.float16(1.0 + 2.0 ** -9)
    assert ex.rn16(vals[4]) == np.float16(2.0 ** -14)
    assert ex.rn16(vals[6]) == np.float16(0.0)
    assert ex.rn16(vals[7]) == np.float16(2.0 ** -24)
    assert ex.rn16(vals[9]) == np.float16(65504.0) and np.isinf(ex.rn16(vals[10]))


def test_relative_gap_hand_computed():
    """(runner-up - best) / best over the grid: the quantity that decides when the GPU's alpha*
    must equal the oracle's ([notes] 方法: alpha* = argmin L). Hand-computed values."""
    assert oracle.relative_gap([3.0, 1.0, 1.5, 2.0]) == 0.5
    assert oracle.relative_gap([2.5, 2.0]) == 0.25
    assert oracle.relative_gap([4.0, 1.0, 1.0]) == 0.0          # a tie: no gap
    assert oracle.relative_gap([1.0, 1.25, 4.0]) == 0.25
    assert oracle.relative_gap([0.0, 1.0]) == float("inf")      # a zero loss: any other is worse
    # order-free: the same set in any order
    g = np.random.default_rng(4)
    ls = g.uniform(1.0, 2.0, 20)
    assert oracle.relative_gap(ls) == oracle.relative_gap(ls[::-1])
    srt = np.sort(ls)
    assert oracle.relative_gap(ls) == (srt[1] - srt[0]) / srt[0]


def test_accuracy_report_hand_computed():
    """The metrics of "FlashAttention的量化：INT8和FP8怎么用才不影响精度？", section 精度验证 (max
    abs, max rel, mean abs) and the relative Frobenius error of the W4A16 bar, on a case worked
    by hand: test [1, 2, 3.5, 0.25], reference [1, 2.5, 3, 0]."""
    r = oracle.accuracy_report(np.array([1.0, 2.0, 3.5, 0.25]), np.array([1.0, 2.5, 3.0, 0.0]))
    assert r["max_abs"] == 0.5
    # relative errors 0, 0.2, 1/6 and 0.25 / 1e-6 (|ref| clamped at 1e-6)
    assert r["max_rel"] == pytest.approx(0.25 / 1e-6, rel=1e-15)
    assert r["mean_abs"] == pytest.approx((0.0 + 0.5 + 0.5 + 0.25) / 4, rel=1e-15)
    assert r["rel_fro"] == pytest.approx(math.sqrt(0.25 + 0.25 + 0.0625) / math.sqrt(1 + 6.25 + 9),
                                         rel=1e-15)
    r = oracle.accuracy_report(np.array([[3.0, 4.0]]), np.array([[0.0, 0.0]]))
    assert r["rel_fro"] == pytest.approx(5.0 / 1e-300, rel=1e-12)   # a zero reference
    r = oracle.accuracy_report(np.array([1.0, -2.0]), np.array([1.0, -2.0]))
    assert r["max_abs"] == 0.0 and r["rel_fro"] == 0.0
