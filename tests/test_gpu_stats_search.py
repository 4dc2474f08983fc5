"""awq_stats_search_layer (s_X and the search in one call) against the two calls it replaces,
awq_act_stats then awq_search_layer, on the same seeded inputs, and s_X against the oracle.

Bars: s_X bit-exact (oracle and act_stats); losses, alpha*, s_best and flags identical to the
two-call path (the search after s_X runs the same kernels on the same s_X). In the Gram form
with fp16 X the column sums come out of the transpose pass, in other dtypes and in the direct
form from the statistics pass. The profiled forms (stage_ms) must give the same results.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import post_weight_quantization_channel_amd as m   # fails loudly if libawq.so is missing
    from post_weight_quantization_channel_amd import _lib
    _lib.load()
    return m


def _layer(seed, n, k, m, xdt=np.float16):
    L = workloads.c2_like_layer(n=n, k=k, m=m, config=seed)
    return L.W, L.X.astype(xdt)


CASES = [
    # name, builder -> (W, X as numpy), torch dtype of X
    ("f16_384x512_m700", lambda: _layer(41, 384, 512, 700), torch.float16),
    ("f16_1x128_m1", lambda: _layer(42, 1, 128, 1), torch.float16),
    ("f16_96x1152_m300", lambda: _layer(43, 96, 1152, 300), torch.float16),
    # 17 chunks of 256 tokens, the last one of 37
    ("f16_320x256_m4133", lambda: _layer(44, 320, 256, 4133), torch.float16),
    ("f32_c1_512x512_m256", lambda: (workloads.c1_layer().W, workloads.c1_layer().X),
     torch.float32),
    ("bf16_320x256_m513", lambda: _layer(45, 320, 256, 513, np.float32), torch.bfloat16),
]


@pytest.mark.parametrize("form", ("direct", "gram"))
@pytest.mark.parametrize("name,make,tdt", CASES, ids=[c[0] for c in CASES])
def test_stats_search_equals_stats_then_search(awq, name, make, tdt, form):
    W, X = make()
    print("   stats_search_layer", name, form, W.shape, X.shape, tdt, flush=True)
    Wt = torch.from_numpy(np.ascontiguousarray(W)).cuda()
    Xt = torch.from_numpy(np.ascontiguousarray(X)).cuda().to(tdt)
    Xref = Xt.float().cpu().numpy() if tdt == torch.bfloat16 else X
    cfg = awq.AwqConfig(form=form)

    sx_f, rf = awq.stats_search_layer(Wt, Xt, cfg)
    sx_s, fl = awq.act_stats(Xt)
    rs = awq.search_layer(Wt, Xt, sx_s, cfg, flags=fl)
    torch.cuda.synchronize()

    sx_f_h = sx_f.cpu().numpy()
    assert np.array_equal(sx_f_h, sx_s.cpu().numpy())
    assert np.array_equal(sx_f_h, oracle.act_stats(Xref))
    assert np.array_equal(rf.losses.cpu().numpy(), rs.losses.cpu().numpy())
    assert int(rf.best.item()) == int(rs.best.item())
    assert np.array_equal(rf.s_best.cpu().numpy(), rs.s_best.cpu().numpy())
    assert int(rf.flags.item()) == int(rs.flags.item()) == 0

    # the profiled form: same results, stage durations filled in
    st = {}
    sx_p, rp = awq.stats_search_layer(Wt, Xt, cfg, stage_ms=st)
    assert np.array_equal(sx_p.cpu().numpy(), sx_f_h)
    assert np.array_equal(rp.losses.cpu().numpy(), rs.losses.cpu().numpy())
    assert int(rp.best.item()) == int(rs.best.item())
    assert all(v >= 0.0 for v in st.values())
    assert st["x_prep"] > 0.0 and st["loss"] > 0.0 and st["quantize_stack"] > 0.0
    if form == "gram":
        assert st["gram_gemm"] > 0.0 and st["gram_finish"] > 0.0
    else:
        assert st["gram_gemm"] == 0.0 or st["gram_gemm"] < 0.01


def test_profiled_search_matches_the_plain_call(awq):
    W, X = _layer(46, 384, 512, 700)
    print("   search_layer profiled vs plain", W.shape, X.shape, flush=True)
    Wt, Xt = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    for form in ("direct", "gram"):
        cfg = awq.AwqConfig(form=form)
        sx, _ = awq.act_stats(Xt)
        r = awq.search_layer(Wt, Xt, sx, cfg)
        st = {}
        rp = awq.search_layer(Wt, Xt, sx, cfg, stage_ms=st)
        assert np.array_equal(r.losses.cpu().numpy(), rp.losses.cpu().numpy())
        assert np.array_equal(r.s_best.cpu().numpy(), rp.s_best.cpu().numpy())
        assert st["scale_table"] > 0.0 and st["loss"] > 0.0 and st["finalize"] > 0.0
        if form == "gram":
            assert st["x_prep"] > 0.0 and st["gram_gemm"] > 0.0 and st["gram_finish"] > 0.0


def test_clip_after_stats_search(awq):
    """The Gram operand the fused call leaves in its workspace serves awq_clip_search_gram as the
    plain search's does."""
    W, X = _layer(47, 256, 512, 900)
    print("   clip_search_gram after stats_search_layer", W.shape, X.shape, flush=True)
    Wt, Xt = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    cfg = awq.AwqConfig(form="gram")
    nbytes = awq.search_workspace_bytes(X.shape[0], W.shape[0], W.shape[1], torch.float16, cfg)
    ws1 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    _, rf = awq.stats_search_layer(Wt, Xt, cfg, workspace=ws1)
    sx, _ = awq.act_stats(Xt)
    rs = awq.search_layer(Wt, Xt, sx, cfg, workspace=ws2)
    c1 = awq.clip_search_gram(Wt, rf.s_best, ws1, cfg)
    c2 = awq.clip_search_gram(Wt, rs.s_best, ws2, cfg)
    torch.cuda.synchronize()
    assert np.array_equal(c1.clip.cpu().numpy(), c2.clip.cpu().numpy())
    assert int(c1.flags.item()) == 0


def test_stats_search_flags(awq):
    """The fused call raises the statistics pass's flags: fp16 column sums of 2^29 or more
    (no longer exact) and a non-finite activation."""
    from post_weight_quantization_channel_amd import _lib as L
    rng = np.random.default_rng(48)
    W = (0.02 * rng.standard_normal((64, 128))).astype(np.float16)
    Xb = rng.standard_normal((9000, 128)).astype(np.float16)
    Xb[:, 5] = 60000.0                      # 9000 * 60000 > 2^29
    print("   stats_search_layer flags", W.shape, Xb.shape, flush=True)
    for form in ("direct", "gram"):
        cfg = awq.AwqConfig(form=form)
        _, r = awq.stats_search_layer(torch.from_numpy(W).cuda(), torch.from_numpy(Xb).cuda(), cfg)
        assert int(r.flags.item()) & L.FLAG_STATS_INEXACT, form
        Xi = Xb.copy()
        Xi[:, 5] = 1.0
        Xi[3, 9] = np.inf
        _, r = awq.stats_search_layer(torch.from_numpy(W).cuda(), torch.from_numpy(Xi).cuda(), cfg)
        assert int(r.flags.item()) & L.FLAG_NONFINITE_X, form


@pytest.mark.parametrize("form", ("direct", "gram"))
def test_stats_search_layers_equals_stats_then_search(awq, form):
    """awq_stats_search_layers against act_stats + search_layers on q/k/v-like weights."""
    g = np.random.default_rng(49)
    X = workloads.c2_like_layer(n=8, k=384, m=700, config=50).X
    Ws = [torch.from_numpy((0.02 * g.standard_normal((n, 384))).astype(np.float16)).cuda()
          for n in (200, 64, 136)]
    print("   stats_search_layers", form, [tuple(W.shape) for W in Ws], X.shape, flush=True)
    Xt = torch.from_numpy(X).cuda()
    cfg = awq.AwqConfig(form=form)
    sx_f, rf = awq.search_layers(Ws, Xt, None, cfg)
    sx_s, fl = awq.act_stats(Xt)
    rs = awq.search_layers(Ws, Xt, sx_s, cfg, flags=fl)
    torch.cuda.synchronize()
    assert np.array_equal(sx_f.cpu().numpy(), sx_s.cpu().numpy())
    assert np.array_equal(sx_f.cpu().numpy(), oracle.act_stats(X))
    assert np.array_equal(rf.losses.cpu().numpy(), rs.losses.cpu().numpy())
    assert int(rf.best.item()) == int(rs.best.item())
    assert np.array_equal(rf.s_best.cpu().numpy(), rs.s_best.cpu().numpy())
    assert int(rf.flags.item()) == int(rs.flags.item()) == 0


def test_whole_path_on_a_side_stream(awq):
    """Every call launches on the caller's stream: the path run under a side stream (torch's
    current stream there) gives the default stream's results bit for bit."""
    W, X = _layer(51, 320, 512, 900)
    print("   whole path on a side stream", W.shape, X.shape, flush=True)
    Wt, Xt = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    A = torch.from_numpy(workloads.w4a16_activations(3, 512, config=5)).cuda()

    def path(form):
        cfg = awq.AwqConfig(form=form)
        sx, r = awq.stats_search_layer(Wt, Xt, cfg)
        p = awq.pack_int4(Wt, r.s_best, cfg, flags=r.flags)
        Y = awq.w4a16_gemm(A, p.qweight, p.scales16, p.s16)
        return [sx, r.losses, r.s_best, p.qweight, p.scales16, Y, r.flags]

    for form in ("direct", "gram"):
        ref = [t.clone() for t in path(form)]
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            out = path(form)
        side.synchronize()
        for a, b in zip(ref, out):
            assert torch.equal(a, b), form
