"""GPU parity of w4a16_gemm_ws (K split over workgroups for M <= 64) against the oracle.

Bar: ||Y_gpu - Y||_F / ||Y||_F <= 2e-3 against the fp64 oracle, as for w4a16_gemm; exact on the
integer case; results bit-identical from call to call and independent of the workspace's
history (the slices are added in a fixed order).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

W4A16_RTOL = 2e-3


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import post_weight_quantization_channel_amd as m   # fails loudly if libawq.so is missing
    from post_weight_quantization_channel_amd import _lib
    _lib.load()
    return m


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(*a):
    print("  ", *a, flush=True)


def _check(Y, A, qw, sc, s, group=128, z=None, rows=None):
    rows = slice(None) if rows is None else rows
    ref = oracle.w4a16(A, qw[rows], sc[rows], s, group=group,
                       zeros=None if z is None else z[rows])
    y = host(Y)[:, rows].astype(np.float64)
    assert np.all(np.isfinite(y))
    rep = oracle.accuracy_report(y, ref)
    say(rep)
    assert rep["rel_fro"] <= W4A16_RTOL


# (n, k, m): the split kernel with 1, 2 and 4 blocks of 16 rows, one and several slices, a ragged
# last slice (K = 11008: 86 blocks in slices of 11), ragged tiles (N % 64, N % 4), one slice
# without a workspace (32768 rows); and shapes the call hands to w4a16_gemm's kernels
WS_CASES = [(384, 512, m) for m in (1, 2, 16, 17, 64)] + \
           [(4096, 4096, m) for m in (1, 16, 33, 64)] + \
           [(11008, 4096, m) for m in (16, 17, 32, 64)] + \
           [(4096, 11008, 16), (4096, 8192, 20), (2048, 8192, 16), (1024, 28672, 2),
            (130, 1024, 40), (1002, 2048, 64), (130, 32768, 48), (32768, 4096, 48),
            (8192, 4096, 24)] + \
           [(4096, 4096, 128), (4096, 4096, 65), (11008, 4096, 128), (4096, 11008, 100),
            (130, 2048, 67), (1002, 4096, 300), (130, 32768, 200), (4096, 4096, 512)]


@pytest.mark.parametrize("n,k,m", WS_CASES)
def test_w4a16_ws_parity(awq, n, k, m):
    qw, sc, s = workloads.w4a16_random_artifacts(n, k, config=4, j=n + m)
    A = workloads.w4a16_activations(m, k, config=4, j=n + m)
    say("w4a16_ws", (m, k), "x", (n, k), "workspace", awq.w4a16_gemm_workspace_bytes(m, n, k))
    Y = awq.w4a16_gemm_ws(dev(A), dev(qw.view(np.int32)), dev(sc), dev(s))
    _check(Y, A, qw, sc, s, rows=slice(0, min(n, 2048)))


WS_VARIANTS = [(g, zp, hs) for g in (128, 64) for zp in (False, True) for hs in (True, False)]


@pytest.mark.parametrize("group,zp,with_s", WS_VARIANTS)
@pytest.mark.parametrize("n,k,m", [(320, 8192, 16), (4096, 4096, 40), (1000, 11008, 20),
                                   (1000, 4096, 100)])
def test_w4a16_ws_group_zero_point_and_folded_s(awq, group, zp, with_s, n, k, m):
    qw, sc, s = workloads.w4a16_random_artifacts(n, k, group=group, config=4, j=n + m)
    z = workloads.w4a16_random_zeros(n, k, group=group, config=4, j=n + m) if zp else None
    A = workloads.w4a16_activations(m, k, config=4, j=n + m)
    s_eff = s if with_s else np.ones_like(s)
    say("w4a16_ws", (m, k), "x", (n, k), "group", group, "zero point", zp, "s", with_s)
    Y = awq.w4a16_gemm_ws(dev(A), dev(qw.view(np.int32)), dev(sc),
                          dev(s) if with_s else None, group=group,
                          zeros=None if z is None else dev(z))
    _check(Y, A, qw, sc, s_eff, group=group, z=z)


def test_w4a16_ws_exact_integer_case(awq):
    """Unit steps and s, small integer activations: every partial sum is an integer below 2^24,
    so the split sums and the fp16 output are exact."""
    g = np.random.default_rng(45)
    q = g.integers(-8, 8, size=(272, 2048), dtype=np.int8)
    qw = oracle.pack_int4(q)
    A = g.integers(-3, 4, size=(37, 2048)).astype(np.float16)
    sc = np.ones((272, 16), np.float16)
    s = np.ones(2048, np.float16)
    assert awq.w4a16_gemm_workspace_bytes(37, 272, 2048) > 0       # several slices
    say("w4a16_ws exact integers")
    Y = awq.w4a16_gemm_ws(dev(A), dev(qw.view(np.int32)), dev(sc), dev(s))
    ref = oracle.w4a16(A, qw, sc, s)
    assert np.array_equal(host(Y).astype(np.float64), ref)


def test_w4a16_ws_reuse_and_determinism(awq):
    """One explicit workspace for calls in a row, the second with fewer rows and another shape:
    every result equals, bit for bit, that of the same call on a fresh workspace filled with
    other bytes."""
    from post_weight_quantization_channel_amd import _lib
    shapes = [(4096, 4096, 128), (4096, 4096, 64), (1024, 8192, 16), (4096, 4096, 128)]
    need = max(awq.w4a16_gemm_workspace_bytes(m, n, k) for n, k, m in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws.fill_(0x5A)
    for i, (n, k, m) in enumerate(shapes):
        qw, sc, s = workloads.w4a16_random_artifacts(n, k, config=4, j=7 + n)
        A = workloads.w4a16_activations(m, k, config=4, j=7 + n)
        args = (dev(A), dev(qw.view(np.int32)), dev(sc), dev(s))
        say("w4a16_ws reuse", i, (m, k), "x", (n, k))
        Y1 = host(awq.w4a16_gemm_ws(*args, workspace=ws))
        fresh = torch.full((need,), 0xC3, dtype=torch.uint8, device="cuda")
        Y2 = host(awq.w4a16_gemm_ws(*args, workspace=fresh))
        assert np.array_equal(Y1.view(np.uint16), Y2.view(np.uint16))
        if i == 0:
            _check(torch.from_numpy(Y1), A, qw, sc, s, rows=slice(0, 1024))
    # a workspace that is too small is refused before anything runs
    n, k, m = shapes[0]
    qw, sc, s = workloads.w4a16_random_artifacts(n, k, config=4, j=1)
    A = workloads.w4a16_activations(m, k, config=4, j=1)
    with pytest.raises(_lib.AwqError):
        awq.w4a16_gemm_ws(dev(A), dev(qw.view(np.int32)), dev(sc), dev(s), workspace=ws[:1024])


def _fuzz_cases(n_cases=16, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n_cases):
        n = int(g.choice([int(g.integers(1, 300)), int(g.integers(300, 20000))]))
        k = 128 * int(g.integers(1, 97))
        m = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 300))]))
        out.append((i, n, k, m, int(g.choice([64, 128])), bool(g.integers(0, 2)),
                    bool(g.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,n,k,m,group,zp,with_s", _fuzz_cases())
def test_w4a16_ws_fuzz(awq, i, n, k, m, group, zp, with_s):
    """Seeded random shapes (ragged N and M, K up to 12288), groups, codes and s: both entry
    points against the oracle on the first 512 rows."""
    qw, sc, s = workloads.w4a16_random_artifacts(n, k, group=group, config=4, j=100 + i)
    z = workloads.w4a16_random_zeros(n, k, group=group, config=4, j=100 + i) if zp else None
    A = workloads.w4a16_activations(m, k, config=4, j=100 + i)
    s_eff = s if with_s else np.ones_like(s)
    say("w4a16 fuzz", i, (m, k), "x", (n, k), "group", group, "zero point", zp, "s", with_s,
        "workspace", awq.w4a16_gemm_workspace_bytes(m, n, k, group))
    args = (dev(A), dev(qw.view(np.int32)), dev(sc), dev(s) if with_s else None)
    kw = dict(group=group, zeros=None if z is None else dev(z))
    rows = slice(0, min(n, 512))
    _check(awq.w4a16_gemm_ws(*args, **kw), A, qw, sc, s_eff, group=group, z=z, rows=rows)
    _check(awq.w4a16_gemm(*args, **kw), A, qw, sc, s_eff, group=group, z=z, rows=rows)
