"""The C-ABI library loads, exports every call include/awq.h declares, and rejects bad arguments
with the documented status before any HIP call (these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

from post_weight_quantization_channel_amd import _lib  # noqa: E402
from post_weight_quantization_channel_amd._lib import AwqCfg  # noqa: E402

FAKE = 0x10000        # aligned, never dereferenced: every call below fails validation first
FAKE2 = 0x20000


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("awq_act_stats", "awq_search_layer", "awq_pack_int4", "w4a16_gemm",
              "w4a16_gemm_ws", "w4a16_gemm_workspace_bytes",
              "awq_search_workspace_bytes", "awq_act_stats_workspace_bytes",
              "awq_clip_search", "awq_clip_workspace_bytes", "awq_search_layers",
              "awq_clip_search_gram", "awq_clip_search_gram_ws_bytes",
              "awq_fold_scale", "awq_stats_search_layer", "awq_search_layer_profiled",
              "awq_stats_search_layers",
              "awq_status_string", "awq_version"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(7):
        s = lib.awq_status_string(code).decode()
        assert s.startswith("AWQ_")
    assert lib.awq_version() == 10700


def cfg(bits=4, group=128, n_grid=20, s_floor=1e-5, form=0, n_clip=11, clip_min=0.5,
        zero_point=0):
    return AwqCfg(bits, group, n_grid, s_floor, form, n_clip, clip_min, zero_point)


def test_workspace_queries(lib):
    # stats: one fp64 partial and one exponent byte per (256-row chunk, column)
    assert lib.awq_act_stats_workspace_bytes(65536, 4096) == 256 * 4096 * 9
    assert lib.awq_act_stats_workspace_bytes(300, 72) == 1280 + 256   # each part 256-aligned
    assert lib.awq_act_stats_workspace_bytes(0, 4096) == 0
    ws = lib.awq_search_workspace_bytes(65536, 4096, 4096, _lib.AWQ_F16, cfg())
    estack = 20 * 4096 * 4096 * 2
    assert estack < ws < estack + 4 * 2**20
    ws32 = lib.awq_search_workspace_bytes(256, 512, 512, _lib.AWQ_F32, cfg())
    assert ws32 >= 256 * 512 * 2 + 20 * 512 * 512 * 2
    assert lib.awq_search_workspace_bytes(256, 512, 512, _lib.AWQ_F16, cfg(bits=5)) == 0
    assert lib.awq_search_workspace_bytes(256, 512, 512, _lib.AWQ_F16, cfg(n_grid=1)) == 0
    assert lib.awq_search_workspace_bytes(256, 512, 512, _lib.AWQ_F16, cfg(form=2)) == 0
    # fewer than 256 rows or tokens: an fp32 error stack and no fp16 copy of X
    small = lib.awq_search_workspace_bytes(4096, 255, 1024, _lib.AWQ_F32, cfg())
    assert 20 * 255 * 1024 * 4 < small < 20 * 255 * 1024 * 4 + 2**20
    small = lib.awq_search_workspace_bytes(255, 512, 1024, _lib.AWQ_F32, cfg())
    assert 20 * 512 * 1024 * 4 < small < 20 * 512 * 1024 * 4 + 2**20


def _gram_chunks(M, K):
    """Token chunks of X^T X: (tile, chunk) workgroups should fill whole waves of 256 CUs, so
    the count minimises ceil(tiles * chunks / 256) * chunk_length (chunks of a multiple of 128
    tokens, at most 32 chunks and 4096 workgroups; ties go to fewer chunks)."""
    t = -(-K // 256)
    T = t * (t + 1) // 2
    Mp = -(-M // 128) * 128
    best = None
    for s in range(1, max(1, min(Mp // 128, 32, 4096 // T)) + 1):
        chunk = -(-(-(-Mp // s)) // 128) * 128
        se = -(-Mp // chunk)
        cost = -(-T * se // 256) * chunk
        if best is None or cost < best[0]:
            best = (cost, se)
    return T, best[1]


def test_gram_workspace(lib):
    """Gram form: K x K fp16 operand + d, and one region shared by the error stack and by the
    transposed X plus the fp32 partials of X^T X (one 256 KiB tile per (tile, chunk))."""
    g = cfg(form=_lib.AWQ_FORM_GRAM)
    ws = lib.awq_search_workspace_bytes(65536, 4096, 4096, _lib.AWQ_F16, g)
    T, S = _gram_chunks(65536, 4096)
    assert T == 136 and S == 13       # 13 chunks of 5120 tokens: 1768 workgroups, 7 waves
    xt = 4096 * 65536 * 2
    hpart = S * T * 256 * 256 * 4
    estack = 20 * 4096 * 4096 * 2
    fixed = 4096 * 4096 * 2
    assert fixed + max(xt + hpart, estack) < ws < fixed + max(xt + hpart, estack) + 4 * 2**20
    # a small layer: the error stack dominates the shared region
    ws_small = lib.awq_search_workspace_bytes(256, 512, 512, _lib.AWQ_F16, g)
    assert 512 * 512 * 2 + 20 * 512 * 512 * 2 < ws_small < 512 * 512 * 2 + 20 * 512 * 512 * 2 + 2**20
    # limits of the Gram form: K <= 32768, padded M < 2^23
    assert lib.awq_search_workspace_bytes(256, 64, 32768 + 128, _lib.AWQ_F16, g) == 0
    assert lib.awq_search_workspace_bytes(256, 64, 32768, _lib.AWQ_F16, g) > 0
    assert lib.awq_search_workspace_bytes((1 << 23) - 128, 64, 256, _lib.AWQ_F16, g) > 0
    assert lib.awq_search_workspace_bytes((1 << 23) - 127, 64, 256, _lib.AWQ_F16, g) == 0


def test_act_stats_rejects(lib):
    f = lib.awq_act_stats
    assert f(None, 1, 4, 8, 8, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_NULL
    assert f(FAKE, 7, 4, 8, 8, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_DTYPE
    assert f(FAKE, 1, 0, 8, 8, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE, 1, 4, 12, 12, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE, 1, 4, 8, 4, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE + 2, 1, 4, 8, 8, FAKE, FAKE, FAKE, 1 << 20, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE, 1, 4, 8, 8, FAKE, FAKE, FAKE, 8, None) == _lib.AWQ_ERR_WORKSPACE
    assert f(FAKE, 1, 4, 8, 8, FAKE, FAKE, None, 1 << 20, None) == _lib.AWQ_ERR_WORKSPACE


def test_act_stats_noalloc_rejects(lib):
    """Host checks of the call that allocates nothing, before any HIP call: the same argument
    rules as awq_act_stats, and shapes whose scratch exceeds the static array's 32 MiB."""
    f = lib.awq_act_stats_noalloc
    assert f(None, 1, 4, 8, 8, FAKE, FAKE, None) == _lib.AWQ_ERR_NULL
    assert f(FAKE, 1, 4, 8, 8, None, FAKE, None) == _lib.AWQ_ERR_NULL
    assert f(FAKE, 7, 4, 8, 8, FAKE, FAKE, None) == _lib.AWQ_ERR_DTYPE
    assert f(FAKE, 1, 0, 8, 8, FAKE, FAKE, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE, 1, 4, 12, 12, FAKE, FAKE, None) == _lib.AWQ_ERR_SHAPE
    assert f(FAKE + 2, 1, 4, 8, 8, FAKE, FAKE, None) == _lib.AWQ_ERR_SHAPE
    lim = _lib.NOALLOC_SCRATCH_BYTES
    # 65536 tokens (256 chunks): K = 14560 fits, 14568 does not
    assert lib.awq_act_stats_workspace_bytes(65536, 14560) <= lim
    assert lib.awq_act_stats_workspace_bytes(65536, 14568) > lim
    assert f(FAKE, 1, 65536, 14568, 14568, FAKE, FAKE, None) == _lib.AWQ_ERR_WORKSPACE
    assert f(FAKE, 1, 1 << 20, 4096, 4096, FAKE, FAKE, None) == _lib.AWQ_ERR_WORKSPACE


def _search(lib, **kw):
    a = dict(W=FAKE, wdt=1, N=256, K=512, X=FAKE2, xdt=1, M=300, sx=FAKE, cfg=cfg(),
             losses=FAKE, best=FAKE, s_best=FAKE, flags=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    c = a["cfg"]
    return lib.awq_search_layer(a["W"], a["wdt"], a["N"], a["K"], a["X"], a["xdt"], a["M"],
                                a["sx"], ctypes.byref(c) if c is not None else None,
                                a["losses"], a["best"], a["s_best"], a["flags"], a["ws"],
                                a["ws_bytes"], None)


def test_search_rejects(lib):
    E = _lib
    for k in ("W", "X", "sx", "losses", "best", "s_best", "flags"):
        assert _search(lib, **{k: None}) == E.AWQ_ERR_NULL, k
    assert _search(lib, cfg=None) == E.AWQ_ERR_NULL
    assert _search(lib, cfg=cfg(bits=2)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(group=32)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(zero_point=3)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(n_grid=1)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(n_grid=65)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(s_floor=0.0)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(s_floor=float("nan"))) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(form=2)) == E.AWQ_ERR_CONFIG
    assert _search(lib, cfg=cfg(form=-1)) == E.AWQ_ERR_CONFIG
    gram = cfg(form=E.AWQ_FORM_GRAM)
    assert _search(lib, cfg=gram, K=32768 + 128) == E.AWQ_ERR_SHAPE
    assert _search(lib, cfg=gram, M=(1 << 23) - 127) == E.AWQ_ERR_SHAPE
    need_g = lib.awq_search_workspace_bytes(300, 256, 512, 1, gram)
    assert _search(lib, cfg=gram, ws_bytes=need_g - 1) == E.AWQ_ERR_WORKSPACE
    assert _search(lib, wdt=2) == E.AWQ_ERR_DTYPE      # bf16 W is not accepted
    assert _search(lib, xdt=9) == E.AWQ_ERR_DTYPE
    assert _search(lib, K=500) == E.AWQ_ERR_SHAPE
    assert _search(lib, K=64) == E.AWQ_ERR_SHAPE
    assert _search(lib, K=(1 << 22) + 128) == E.AWQ_ERR_SHAPE
    assert _search(lib, M=0) == E.AWQ_ERR_SHAPE
    assert _search(lib, N=0) == E.AWQ_ERR_SHAPE
    assert _search(lib, W=FAKE + 4) == E.AWQ_ERR_SHAPE
    assert _search(lib, ws=None) == E.AWQ_ERR_WORKSPACE
    need = lib.awq_search_workspace_bytes(300, 256, 512, 1, cfg())
    assert _search(lib, ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE


def _stats_search(lib, **kw):
    a = dict(W=FAKE, wdt=1, N=256, K=512, X=FAKE2, xdt=1, M=300, cfg=cfg(), sx=FAKE,
             losses=FAKE, best=FAKE, s_best=FAKE, flags=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    c = a["cfg"]
    return lib.awq_stats_search_layer(a["W"], a["wdt"], a["N"], a["K"], a["X"], a["xdt"], a["M"],
                                      ctypes.byref(c) if c is not None else None, a["sx"],
                                      a["losses"], a["best"], a["s_best"], a["flags"], a["ws"],
                                      a["ws_bytes"], None, None)


def test_stats_search_rejects(lib):
    E = _lib
    for k in ("W", "X", "sx", "losses", "best", "s_best", "flags"):
        assert _stats_search(lib, **{k: None}) == E.AWQ_ERR_NULL, k
    assert _stats_search(lib, cfg=None) == E.AWQ_ERR_NULL
    assert _stats_search(lib, cfg=cfg(bits=5)) == E.AWQ_ERR_CONFIG
    assert _stats_search(lib, xdt=9) == E.AWQ_ERR_DTYPE
    assert _stats_search(lib, K=500) == E.AWQ_ERR_SHAPE
    assert _stats_search(lib, M=0) == E.AWQ_ERR_SHAPE
    # more than 65535 chunks of 256 tokens for the statistics pass
    assert _stats_search(lib, M=256 * 65535 + 1, N=1, K=128) == E.AWQ_ERR_SHAPE
    assert _stats_search(lib, ws=None) == E.AWQ_ERR_WORKSPACE
    for form in (E.AWQ_FORM_DIRECT, E.AWQ_FORM_GRAM):
        c = cfg(form=form)
        need = lib.awq_search_workspace_bytes(300, 256, 512, 1, c)
        assert _stats_search(lib, cfg=c, ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE


def test_search_workspace_holds_the_statistics_partials(lib):
    # one token and few channels: the statistics' chunk partials (fp64 [1][K]) still fit in the
    # region they share (the direct form's error stack is only n_grid * N * K fp16)
    for form in (_lib.AWQ_FORM_DIRECT, _lib.AWQ_FORM_GRAM):
        for M, N, K in ((1, 1, 128), (65536, 1, 128), (300, 3, 256)):
            need = lib.awq_search_workspace_bytes(M, N, K, 1, cfg(form=form, n_grid=2))
            assert need >= ((M + 255) // 256) * K * 8


def test_pack_rejects(lib):
    E = _lib
    c = cfg()
    f = lib.awq_pack_int4

    def call(W=FAKE, wdt=1, N=4, K=128, s=FAKE, clip=None, cfg_=c, zeros=None, codes=None):
        return f(W, wdt, N, K, s, clip, cfg_, FAKE, FAKE, zeros, FAKE, codes, FAKE, None)
    assert call(W=None) == E.AWQ_ERR_NULL
    assert call(cfg_=None) == E.AWQ_ERR_NULL
    assert call(cfg_=cfg(bits=8)) == E.AWQ_ERR_CONFIG
    assert call(cfg_=cfg(group=32)) == E.AWQ_ERR_CONFIG
    assert call(cfg_=cfg(zero_point=2)) == E.AWQ_ERR_CONFIG
    assert call(cfg_=cfg(zero_point=1)) == E.AWQ_ERR_NULL       # zeros required
    assert call(zeros=FAKE) == E.AWQ_ERR_CONFIG                 # zeros without zero points
    assert call(wdt=2) == E.AWQ_ERR_DTYPE
    assert call(K=130) == E.AWQ_ERR_SHAPE
    assert call(K=192) == E.AWQ_ERR_SHAPE                        # not a multiple of 128
    assert call(K=64, cfg_=cfg(group=64)) == E.AWQ_ERR_SHAPE     # K below 128
    assert call(K=160, cfg_=cfg(group=64)) == E.AWQ_ERR_SHAPE
    assert call(N=0) == E.AWQ_ERR_SHAPE
    assert call(codes=FAKE + 3) == E.AWQ_ERR_SHAPE
    assert call(clip=FAKE + 2) == E.AWQ_ERR_SHAPE


def test_group64_and_zero_point_configs_are_accepted(lib):
    """Workspace queries accept group 64 (K a multiple of 64, at least 128) and zero points."""
    for g, zp in ((64, 0), (64, 1), (128, 1)):
        assert lib.awq_search_workspace_bytes(300, 256, 192 if g == 64 else 256, 1,
                                              cfg(group=g, zero_point=zp)) > 0
        assert lib.awq_clip_workspace_bytes(300, 256, 320 if g == 64 else 384, 1,
                                            cfg(group=g, zero_point=zp)) > 0
    assert lib.awq_search_workspace_bytes(300, 256, 64, 1, cfg(group=64)) == 0
    assert lib.awq_search_workspace_bytes(300, 256, 192, 1, cfg(group=128)) == 0


def _clip(lib, **kw):
    a = dict(W=FAKE, wdt=1, N=256, K=512, X=FAKE2, xdt=1, M=300, s=FAKE, cfg=cfg(), clip=FAKE,
             err=None, flags=FAKE, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    c = a["cfg"]
    return lib.awq_clip_search(a["W"], a["wdt"], a["N"], a["K"], a["X"], a["xdt"], a["M"],
                               a["s"], ctypes.byref(c) if c is not None else None, a["clip"],
                               a["err"], a["flags"], a["ws"], a["ws_bytes"], None)


def test_clip_search_rejects(lib):
    E = _lib
    for k in ("W", "X", "s", "clip", "flags"):
        assert _clip(lib, **{k: None}) == E.AWQ_ERR_NULL, k
    assert _clip(lib, cfg=None) == E.AWQ_ERR_NULL
    assert _clip(lib, cfg=cfg(n_clip=1)) == E.AWQ_ERR_CONFIG
    assert _clip(lib, cfg=cfg(n_clip=65)) == E.AWQ_ERR_CONFIG
    assert _clip(lib, cfg=cfg(clip_min=0.0)) == E.AWQ_ERR_CONFIG
    assert _clip(lib, cfg=cfg(clip_min=1.0)) == E.AWQ_ERR_CONFIG
    assert _clip(lib, cfg=cfg(bits=5)) == E.AWQ_ERR_CONFIG
    assert _clip(lib, wdt=2) == E.AWQ_ERR_DTYPE
    assert _clip(lib, xdt=7) == E.AWQ_ERR_DTYPE
    assert _clip(lib, K=500) == E.AWQ_ERR_SHAPE
    assert _clip(lib, M=(1 << 23) - 127) == E.AWQ_ERR_SHAPE
    assert _clip(lib, s=FAKE + 4) == E.AWQ_ERR_SHAPE
    assert _clip(lib, ws=None) == E.AWQ_ERR_WORKSPACE
    need = lib.awq_clip_workspace_bytes(300, 256, 512, 1, cfg())
    # d (fp64 + fp32), two diagonal 256x256 fp16 blocks, X^T fp16 [512, 384] and the partials
    assert need >= 512 * 12 + 2 * 65536 * 2 + 512 * 384 * 2 + 2 * 65536 * 4
    assert _clip(lib, ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE
    assert lib.awq_clip_workspace_bytes(300, 256, 512, 1, cfg(clip_min=2.0)) == 0


def _clip_gram(lib, **kw):
    a = dict(W=FAKE, wdt=1, N=256, K=512, s=FAKE, cfg=cfg(form=1), ws=FAKE2, ws_bytes=1 << 40,
             clip=FAKE, err=None, flags=FAKE)
    a.update(kw)
    c = a["cfg"]
    return lib.awq_clip_search_gram(a["W"], a["wdt"], a["N"], a["K"], a["s"],
                                    ctypes.byref(c) if c is not None else None, a["ws"],
                                    a["ws_bytes"], a["clip"], a["err"], a["flags"], None)


def test_clip_search_gram_rejects(lib):
    E = _lib
    for k in ("W", "s", "clip", "flags", "ws"):
        assert _clip_gram(lib, **{k: None}) == E.AWQ_ERR_NULL, k
    assert _clip_gram(lib, cfg=None) == E.AWQ_ERR_NULL
    assert _clip_gram(lib, cfg=cfg(form=0)) == E.AWQ_ERR_CONFIG      # needs a Gram-form search
    assert _clip_gram(lib, cfg=cfg(form=1, n_clip=1)) == E.AWQ_ERR_CONFIG
    assert _clip_gram(lib, wdt=2) == E.AWQ_ERR_DTYPE
    assert _clip_gram(lib, K=500) == E.AWQ_ERR_SHAPE
    assert _clip_gram(lib, K=32768 + 128) == E.AWQ_ERR_SHAPE
    assert _clip_gram(lib, N=0) == E.AWQ_ERR_SHAPE
    assert _clip_gram(lib, s=FAKE + 4) == E.AWQ_ERR_SHAPE
    need = lib.awq_clip_search_gram_ws_bytes(512, cfg(form=1))
    # the operand sits after the control block, the scale table and d: at least K^2 fp16 in all
    assert need >= 512 * 512 * 2 + 20 * 512 * 4 + 512 * 12
    # it lies inside a Gram-form search workspace of any M and N for this K and n_grid
    for (M, N) in ((128, 1), (300, 256), (65536, 4096)):
        assert lib.awq_search_workspace_bytes(M, N, 512, 1, cfg(form=1)) >= need
    assert _clip_gram(lib, ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE
    assert _clip_gram(lib, ws=FAKE2 + 8) == E.AWQ_ERR_WORKSPACE
    assert lib.awq_clip_search_gram_ws_bytes(512, cfg(form=0)) == 0
    assert lib.awq_clip_search_gram_ws_bytes(500, cfg(form=1)) == 0


def test_search_layers_rejects(lib):
    E = _lib
    P = ctypes.c_void_p
    I64 = ctypes.c_int64

    def call(ptrs=(FAKE, FAKE + 4096), rows=(100, 60), n_w=None, **kw):
        a = dict(wdt=1, K=512, X=FAKE2, xdt=1, M=300, sx=FAKE, cfg=cfg(), losses=FAKE,
                 best=FAKE, s_best=FAKE, flags=FAKE, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        n = len(ptrs) if n_w is None else n_w
        pa = (P * max(1, len(ptrs)))(*ptrs)
        ra = (I64 * max(1, len(rows)))(*rows)
        c = a["cfg"]
        return lib.awq_search_layers(pa, ra, n, a["wdt"], a["K"], a["X"], a["xdt"], a["M"],
                                     a["sx"], ctypes.byref(c) if c is not None else None,
                                     a["losses"], a["best"], a["s_best"], a["flags"], a["ws"],
                                     a["ws_bytes"], None)
    assert call(ptrs=(FAKE, None)) == E.AWQ_ERR_NULL
    assert call(n_w=0) == E.AWQ_ERR_SHAPE
    assert call(ptrs=(FAKE,) * 65, rows=(10,) * 65) == E.AWQ_ERR_SHAPE
    assert call(rows=(100, 0)) == E.AWQ_ERR_SHAPE
    assert call(ptrs=(FAKE, FAKE + 8)) == E.AWQ_ERR_SHAPE       # misaligned second weight
    assert call(cfg=cfg(bits=2)) == E.AWQ_ERR_CONFIG
    need = lib.awq_search_workspace_bytes(300, 160, 512, 1, cfg())
    assert call(ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE
    assert lib.awq_search_layers(None, None, 1, 1, 512, FAKE2, 1, 300, FAKE,
                                 ctypes.byref(cfg()), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                 None) == E.AWQ_ERR_NULL


def test_stats_search_layers_rejects(lib):
    E = _lib
    P = ctypes.c_void_p
    I64 = ctypes.c_int64

    def call(ptrs=(FAKE, FAKE + 4096), rows=(100, 60), **kw):
        a = dict(wdt=1, K=512, X=FAKE2, xdt=1, M=300, cfg=cfg(), sx=FAKE, losses=FAKE,
                 best=FAKE, s_best=FAKE, flags=FAKE, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        pa = (P * len(ptrs))(*ptrs)
        ra = (I64 * len(rows))(*rows)
        c = a["cfg"]
        return lib.awq_stats_search_layers(pa, ra, len(ptrs), a["wdt"], a["K"], a["X"], a["xdt"],
                                           a["M"], ctypes.byref(c) if c is not None else None,
                                           a["sx"], a["losses"], a["best"], a["s_best"],
                                           a["flags"], a["ws"], a["ws_bytes"], None)
    assert call(sx=None) == E.AWQ_ERR_NULL
    assert call(ptrs=(FAKE, None)) == E.AWQ_ERR_NULL
    assert call(cfg=cfg(bits=2)) == E.AWQ_ERR_CONFIG
    assert call(M=256 * 65535 + 1, K=128, rows=(1, 1)) == E.AWQ_ERR_SHAPE
    need = lib.awq_search_workspace_bytes(300, 160, 512, 1, cfg())
    assert call(ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE


def test_fold_scale_rejects(lib):
    E = _lib
    f = lib.awq_fold_scale
    assert f(None, 1, 1, 64, 64, FAKE, 1, FAKE, None) == E.AWQ_ERR_NULL
    assert f(FAKE, 1, 1, 64, 64, None, 1, FAKE, None) == E.AWQ_ERR_NULL
    assert f(FAKE, 1, 1, 64, 64, FAKE, 1, None, None) == E.AWQ_ERR_NULL
    assert f(FAKE, 5, 1, 64, 64, FAKE, 1, FAKE, None) == E.AWQ_ERR_DTYPE
    assert f(FAKE, 1, 0, 64, 64, FAKE, 1, FAKE, None) == E.AWQ_ERR_SHAPE
    assert f(FAKE, 1, 2, 64, 32, FAKE, 1, FAKE, None) == E.AWQ_ERR_SHAPE     # ld < cols
    assert f(FAKE, 1, 2, 64, 64, FAKE, 2, FAKE, None) == E.AWQ_ERR_SHAPE     # axis
    assert f(FAKE + 1, 1, 2, 64, 64, FAKE, 1, FAKE, None) == E.AWQ_ERR_SHAPE  # fp16 misaligned
    assert f(FAKE + 2, 0, 2, 64, 64, FAKE, 1, FAKE, None) == E.AWQ_ERR_SHAPE  # fp32 misaligned
    assert f(FAKE, 1, 2, 64, 64, FAKE + 2, 1, FAKE, None) == E.AWQ_ERR_SHAPE  # s misaligned


def test_w4a16_rejects(lib):
    E = _lib
    f = lib.w4a16_gemm

    def call(A=FAKE, M=1, N=16, K=128, group=128, qw=FAKE, sc=FAKE, zeros=None, s16=FAKE):
        return f(A, M, N, K, group, qw, sc, zeros, s16, FAKE, None)
    assert call(A=None) == E.AWQ_ERR_NULL
    assert call(qw=None) == E.AWQ_ERR_NULL
    assert call(group=32) == E.AWQ_ERR_CONFIG
    assert call(M=0) == E.AWQ_ERR_SHAPE
    assert call(K=200) == E.AWQ_ERR_SHAPE
    assert call(K=192, group=64) == E.AWQ_ERR_SHAPE              # the kernels step 128 channels
    assert call(K=32768 + 128) == E.AWQ_ERR_SHAPE
    assert call(N=0) == E.AWQ_ERR_SHAPE
    assert call(A=FAKE + 8) == E.AWQ_ERR_SHAPE
    assert call(s16=FAKE + 8) == E.AWQ_ERR_SHAPE


def test_w4a16_ws_rejects(lib):
    E = _lib
    f = lib.w4a16_gemm_ws
    need = lib.w4a16_gemm_workspace_bytes(64, 4096, 4096, 128)

    def call(A=FAKE, M=64, N=4096, K=4096, group=128, qw=FAKE, sc=FAKE, zeros=None, s16=FAKE,
             ws=FAKE, ws_bytes=need):
        return f(A, M, N, K, group, qw, sc, zeros, s16, FAKE, ws, ws_bytes, None)
    assert call(A=None) == E.AWQ_ERR_NULL
    assert call(group=32) == E.AWQ_ERR_CONFIG
    assert call(M=0) == E.AWQ_ERR_SHAPE
    assert call(K=200) == E.AWQ_ERR_SHAPE
    assert call(K=32768 + 128) == E.AWQ_ERR_SHAPE
    assert call(A=FAKE + 8) == E.AWQ_ERR_SHAPE
    assert call(ws=None) == E.AWQ_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == E.AWQ_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == E.AWQ_ERR_WORKSPACE                  # not 16-byte aligned
    assert call(M=128, ws=None) == E.AWQ_ERR_WORKSPACE               # tiled kernel on slices


def test_w4a16_workspace_bytes(lib):
    """The split plan: 64-row tiles, slices of >= 4 blocks, at most 512 workgroups; partials of
    S x tiles x 4 waves x MB x 1 KiB. It is taken above 32 rows, from 17 rows with N >= 8192,
    from 16 rows with K >= 8192; elsewhere no workspace."""
    wsb = lib.w4a16_gemm_workspace_bytes
    # 4096 x 4096: 64 tiles, 8 slices of 4 blocks
    assert wsb(33, 4096, 4096, 128) == 8 * 64 * 4 * 4 * 1024
    assert wsb(64, 4096, 4096, 64) == 8 * 64 * 4 * 4 * 1024
    assert wsb(16, 4096, 4096, 128) == 0 and wsb(32, 4096, 4096, 128) == 0
    # 11008 x 4096: 172 tiles, 2 slices of 16 blocks (3 would be 516 workgroups)
    assert wsb(17, 11008, 4096, 128) == 2 * 172 * 4 * 2 * 1024
    assert wsb(16, 11008, 4096, 128) == 0
    # 1024 x 8192: 16 tiles, 16 slices of 4 blocks
    assert wsb(16, 1024, 8192, 128) == 16 * 16 * 4 * 1024
    assert wsb(15, 1024, 8192, 128) == 0
    # one slice (no workspace): more than 256 tiles, or K of fewer than 8 blocks
    assert wsb(48, 32768, 4096, 128) == 0
    assert wsb(48, 4096, 896, 128) == 0
    # at most 64 blocks per slice: K = 16384 on 1024 tiles still takes two slices
    assert wsb(16, 65536, 16384, 128) == 2 * 1024 * 4 * 1 * 1024
    # one row takes w4a16_gemm's kernel
    assert wsb(1, 1024, 8192, 128) == 0
    # above 64 rows with fewer than 256 tiles: the tiled kernel on S slices of >= 8 steps while
    # tiles * S <= 512; partials [S][M][N] fp32, M N rounded up to a multiple of 4
    assert wsb(128, 4096, 4096, 128) == 4 * 128 * 4096 * 4          # 64 tiles, 4 slices of 8
    assert wsb(65, 4096, 4096, 128) == 4 * 65 * 4096 * 4
    assert wsb(128, 11008, 4096, 128) == 2 * 128 * 11008 * 4        # 172 tiles
    assert wsb(100, 4096, 11008, 64) == 8 * 100 * 4096 * 4          # 86 steps: slices of 11
    assert wsb(67, 130, 1024, 128) == 0                              # 8 steps: one slice
    assert wsb(67, 130, 2048, 128) == 2 * 8712 * 4                   # 67 x 130 = 8710 -> 8712
    assert wsb(512, 11008, 4096, 128) == 0                           # 688 tiles
    assert wsb(512, 4096, 4096, 128) == 0                            # 256 tiles
    assert wsb(16, 4096, 200, 128) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()
