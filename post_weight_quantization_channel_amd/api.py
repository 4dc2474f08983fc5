"""Python face of libawq: the four C-ABI calls on torch tensors.

Argument marshalling only -- torch supplies device memory and the current HIP stream; every step
of the computation runs in the library's HIP kernels. Names follow the C ABI (include/awq.h).
Nothing here synchronises: results are ready when the current stream reaches them.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import AwqCfg, check

_DT = {torch.float32: _lib.AWQ_F32, torch.float16: _lib.AWQ_F16, torch.bfloat16: _lib.AWQ_BF16}


@dataclasses.dataclass(frozen=True)
class AwqConfig:
    """bits in {3, 4}; group = 128 input channels per step; n_grid alpha points i/(n_grid-1);
    s = max(s_X, s_floor)^alpha; form "direct" (contract X with every error matrix) or "gram"
    (form H = X^T X once, then contract each error matrix with H); the clipping search tries
    n_clip ratios from 1 down to clip_min; zero_point selects unsigned codes with a zero point
    per (row, group) instead of symmetric ones; group 128 or 64."""
    bits: int = 4
    group: int = 128
    n_grid: int = 20
    s_floor: float = 1e-5
    form: str = "direct"
    n_clip: int = 11
    clip_min: float = 0.5
    zero_point: bool = False

    def c(self) -> AwqCfg:
        forms = {"direct": _lib.AWQ_FORM_DIRECT, "gram": _lib.AWQ_FORM_GRAM}
        if self.form not in forms:
            raise ValueError(f"form must be one of {sorted(forms)}, got {self.form!r}")
        return AwqCfg(self.bits, self.group, self.n_grid, self.s_floor, forms[self.form],
                      self.n_clip, self.clip_min, int(bool(self.zero_point)))


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _flags(device, flags):
    if flags is None:
        return torch.zeros(1, dtype=torch.int32, device=device)
    return flags


@dataclasses.dataclass
class SearchResult:
    losses: torch.Tensor   # fp64 [n_grid]
    best: torch.Tensor     # int32 [1]
    s_best: torch.Tensor   # fp32 [K]
    flags: torch.Tensor    # int32 [1] holding the uint32 flag bits


@dataclasses.dataclass
class PackResult:
    qweight: torch.Tensor   # int32 [N, K/8] holding the uint32 words
    scales16: torch.Tensor  # fp16 [N, K/group]
    s16: torch.Tensor       # fp16 [K]
    codes: torch.Tensor | None
    flags: torch.Tensor
    zeros: torch.Tensor | None = None   # uint8 [N, K/group] for zero-point codes


def act_stats_workspace_bytes(M: int, K: int) -> int:
    return int(_lib.load().awq_act_stats_workspace_bytes(M, K))


def search_workspace_bytes(M: int, N: int, K: int, x_dtype: torch.dtype, cfg: AwqConfig) -> int:
    c = cfg.c()
    return int(_lib.load().awq_search_workspace_bytes(M, N, K, _DT[x_dtype], c))


def act_stats(X: torch.Tensor, flags: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """s_X = mean over tokens of |X| per input channel (fp32 [K]). X may be a row-strided view
    (unit column stride, row stride a multiple of 8 elements)."""
    lib = _lib.load()
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit column stride")
    M, K = X.shape
    ldx = X.stride(0) if M > 1 else K
    flags = _flags(X.device, flags)
    nbytes = lib.awq_act_stats_workspace_bytes(M, K)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=X.device)
    sx = torch.empty(K, dtype=torch.float32, device=X.device)
    check("awq_act_stats", lib.awq_act_stats(X.data_ptr(), _DT[X.dtype], M, K, ldx, sx.data_ptr(),
                                             flags.data_ptr(), workspace.data_ptr(),
                                             workspace.numel(), _stream(X)))
    return sx, flags


def act_stats_noalloc(X: torch.Tensor, sx: torch.Tensor,
                      flags: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """act_stats into caller-provided sx (fp32 [K]) and flags (int32 [1]) with the library's
    static scratch instead of a workspace: the C call allocates nothing, and neither does this
    binding (usable under graph capture). Overlapping calls on one GPU race."""
    lib = _lib.load()
    if not X.is_cuda or X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be a 2-D device tensor with unit column stride")
    M, K = X.shape
    _dev(sx, "sx")
    _dev(flags, "flags")
    if sx.shape != (K,) or sx.dtype != torch.float32 or flags.numel() != 1 or \
            flags.dtype != torch.int32:
        raise ValueError("sx must be fp32 [K] and flags int32 [1]")
    ldx = X.stride(0) if M > 1 else K
    check("awq_act_stats_noalloc", lib.awq_act_stats_noalloc(
        X.data_ptr(), _DT[X.dtype], M, K, ldx, sx.data_ptr(), flags.data_ptr(), _stream(X)))
    return sx, flags


def search_layer(W: torch.Tensor, X: torch.Tensor, sx: torch.Tensor,
                 cfg: AwqConfig = AwqConfig(), flags: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None,
                 stage_ms: dict | None = None) -> SearchResult:
    """Grid search over alpha: losses L_i, best index, s_best = s_{i*}.

    With a dict as `stage_ms` the profiled C call is used: it fills the dict with the duration
    of each kernel of the search (HIP events on the current stream) and blocks until done."""
    lib = _lib.load()
    for t, nm in ((W, "W"), (X, "X"), (sx, "sx")):
        _dev(t, nm)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or sx.shape != (K,) or sx.dtype != torch.float32:
        raise ValueError("shape mismatch: W [N,K], X [M,K], sx fp32 [K]")
    c = cfg.c()
    flags = _flags(W.device, flags)
    nbytes = lib.awq_search_workspace_bytes(M, N, K, _DT[X.dtype], c)
    if nbytes == 0:
        raise ValueError("invalid shape or config for the search")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    s_best = torch.empty(K, dtype=torch.float32, device=W.device)
    args = (W.data_ptr(), _DT[W.dtype], N, K, X.data_ptr(), _DT[X.dtype], M, sx.data_ptr(), c,
            losses.data_ptr(), best.data_ptr(), s_best.data_ptr(), flags.data_ptr(),
            workspace.data_ptr(), workspace.numel(), _stream(W))
    if stage_ms is None:
        check("awq_search_layer", lib.awq_search_layer(*args))
    else:
        ms = (ctypes.c_float * len(_lib.SEARCH_STAGES))()
        check("awq_search_layer_profiled", lib.awq_search_layer_profiled(*args, ms))
        stage_ms.update({k: float(v) for k, v in zip(_lib.SEARCH_STAGES, ms)})
    return SearchResult(losses, best, s_best, flags)


def stats_search_layer(W: torch.Tensor, X: torch.Tensor, cfg: AwqConfig = AwqConfig(),
                       flags: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       stage_ms: dict | None = None) -> tuple[torch.Tensor, SearchResult]:
    """act_stats and search_layer in one call: returns (s_X, result), s_X identical to what
    act_stats gives for this X. `stage_ms` as in search_layer, with the statistics counted in the
    X preparation stage."""
    lib = _lib.load()
    for t, nm in ((W, "W"), (X, "X")):
        _dev(t, nm)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("shape mismatch: W [N,K], X [M,K]")
    c = cfg.c()
    flags = _flags(W.device, flags)
    nbytes = lib.awq_search_workspace_bytes(M, N, K, _DT[X.dtype], c)
    if nbytes == 0:
        raise ValueError("invalid shape or config for the search")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    sx = torch.empty(K, dtype=torch.float32, device=W.device)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    s_best = torch.empty(K, dtype=torch.float32, device=W.device)
    ms = (ctypes.c_float * len(_lib.SEARCH_STAGES))() if stage_ms is not None else None
    check("awq_stats_search_layer", lib.awq_stats_search_layer(
        W.data_ptr(), _DT[W.dtype], N, K, X.data_ptr(), _DT[X.dtype], M, c, sx.data_ptr(),
        losses.data_ptr(), best.data_ptr(), s_best.data_ptr(), flags.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(W), ms))
    if stage_ms is not None:
        stage_ms.update({k: float(v) for k, v in zip(_lib.SEARCH_STAGES, ms)})
    return sx, SearchResult(losses, best, s_best, flags)


@dataclasses.dataclass
class ClipResult:
    clip: torch.Tensor               # fp32 [N, K/group]: the chosen ratios
    err: torch.Tensor | None         # fp32 [n_clip, N, K/group]: group error of every ratio
    flags: torch.Tensor


def clip_workspace_bytes(M: int, N: int, K: int, x_dtype: torch.dtype, cfg: AwqConfig) -> int:
    return int(_lib.load().awq_clip_workspace_bytes(M, N, K, _DT[x_dtype], cfg.c()))


def clip_search(W: torch.Tensor, X: torch.Tensor, s: torch.Tensor, cfg: AwqConfig = AwqConfig(),
                with_err: bool = False, flags: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> ClipResult:
    """Per (row, group), the clip ratio of the grid whose clipped quantization of W s gives the
    smallest group output error."""
    lib = _lib.load()
    for t, nm in ((W, "W"), (X, "X"), (s, "s")):
        _dev(t, nm)
    N, K = W.shape
    M = X.shape[0]
    if X.shape[1] != K or s.shape != (K,) or s.dtype != torch.float32:
        raise ValueError("shape mismatch: W [N,K], X [M,K], s fp32 [K]")
    c = cfg.c()
    flags = _flags(W.device, flags)
    nbytes = lib.awq_clip_workspace_bytes(M, N, K, _DT[X.dtype], c)
    if nbytes == 0:
        raise ValueError("invalid shape or config for the clipping search")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    G = K // cfg.group
    clip = torch.empty((N, G), dtype=torch.float32, device=W.device)
    err = torch.empty((cfg.n_clip, N, G), dtype=torch.float32, device=W.device) \
        if with_err else None
    check("awq_clip_search", lib.awq_clip_search(
        W.data_ptr(), _DT[W.dtype], N, K, X.data_ptr(), _DT[X.dtype], M, s.data_ptr(), c,
        clip.data_ptr(), err.data_ptr() if err is not None else None, flags.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(W)))
    return ClipResult(clip, err, flags)


def clip_search_gram(W: torch.Tensor, s: torch.Tensor, search_workspace: torch.Tensor,
                     cfg: AwqConfig = AwqConfig(form="gram"), with_err: bool = False,
                     flags: torch.Tensor | None = None) -> ClipResult:
    """The clipping search of clip_search, with H_gg and d taken from the workspace of the
    Gram-form search (search_layer / search_layers with this `cfg` and an explicit workspace)
    that just ran on the same X, instead of being formed from X again."""
    lib = _lib.load()
    _dev(W, "W")
    _dev(s, "s")
    _dev(search_workspace, "search_workspace")
    N, K = W.shape
    if s.shape != (K,) or s.dtype != torch.float32:
        raise ValueError("shape mismatch: W [N,K], s fp32 [K]")
    if cfg.form != "gram":
        raise ValueError("clip_search_gram needs the configuration of a Gram-form search")
    c = cfg.c()
    if lib.awq_clip_search_gram_ws_bytes(K, c) == 0:
        raise ValueError("invalid shape or config for the clipping search")
    flags = _flags(W.device, flags)
    G = K // cfg.group
    clip = torch.empty((N, G), dtype=torch.float32, device=W.device)
    err = torch.empty((cfg.n_clip, N, G), dtype=torch.float32, device=W.device) \
        if with_err else None
    check("awq_clip_search_gram", lib.awq_clip_search_gram(
        W.data_ptr(), _DT[W.dtype], N, K, s.data_ptr(), c, search_workspace.data_ptr(),
        search_workspace.numel() * search_workspace.element_size(), clip.data_ptr(),
        err.data_ptr() if err is not None else None, flags.data_ptr(), _stream(W)))
    return ClipResult(clip, err, flags)


def search_layers(Ws: list, X: torch.Tensor, sx: torch.Tensor | None,
                  cfg: AwqConfig = AwqConfig(), flags: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """One alpha for several weights that read the same X (rows stacked, no copy). With
    sx = None, s_X is taken in the same call (awq_stats_search_layers) and (s_X, result) is
    returned; otherwise the result."""
    lib = _lib.load()
    for i, W in enumerate(Ws):
        _dev(W, f"W[{i}]")
    _dev(X, "X")
    if sx is not None:
        _dev(sx, "sx")
    K = X.shape[1]
    if any(W.shape[1] != K or W.dtype != Ws[0].dtype for W in Ws):
        raise ValueError("every W must be [N_l, K] with the dtype of W[0]")
    Ns = [int(W.shape[0]) for W in Ws]
    M, N = X.shape[0], sum(Ns)
    c = cfg.c()
    flags = _flags(X.device, flags)
    nbytes = lib.awq_search_workspace_bytes(M, N, K, _DT[X.dtype], c)
    if nbytes == 0:
        raise ValueError("invalid shape or config for the search")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    losses = torch.empty(cfg.n_grid, dtype=torch.float64, device=X.device)
    best = torch.empty(1, dtype=torch.int32, device=X.device)
    s_best = torch.empty(K, dtype=torch.float32, device=X.device)
    ptrs = (ctypes.c_void_p * len(Ws))(*[W.data_ptr() for W in Ws])
    rows = (ctypes.c_int64 * len(Ws))(*Ns)
    if sx is None:
        sx_out = torch.empty(K, dtype=torch.float32, device=X.device)
        check("awq_stats_search_layers", lib.awq_stats_search_layers(
            ptrs, rows, len(Ws), _DT[Ws[0].dtype], K, X.data_ptr(), _DT[X.dtype], M, c,
            sx_out.data_ptr(), losses.data_ptr(), best.data_ptr(), s_best.data_ptr(),
            flags.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(X)))
        return sx_out, SearchResult(losses, best, s_best, flags)
    if sx.shape != (K,) or sx.dtype != torch.float32:
        raise ValueError("sx must be fp32 [K]")
    check("awq_search_layers", lib.awq_search_layers(
        ptrs, rows, len(Ws), _DT[Ws[0].dtype], K, X.data_ptr(), _DT[X.dtype], M, sx.data_ptr(),
        c, losses.data_ptr(), best.data_ptr(), s_best.data_ptr(), flags.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream(X)))
    return SearchResult(losses, best, s_best, flags)


def fold_scale(prev: torch.Tensor, s: torch.Tensor, axis: int,
               flags: torch.Tensor | None = None) -> torch.Tensor:
    """In place: prev /= s along `axis` (1: columns of a [rows, K] parameter such as a norm
    weight [1, K]; 0: rows, e.g. a previous linear layer's output channels). Returns flags."""
    lib = _lib.load()
    _dev(s, "s")
    if not prev.is_cuda or prev.dim() != 2 or prev.stride(1) != 1:
        raise ValueError("prev must be a 2-D device tensor with unit column stride")
    rows, cols = prev.shape
    if s.dtype != torch.float32 or s.shape != ((cols,) if axis == 1 else (rows,)):
        raise ValueError("s must be fp32 with one entry per folded channel")
    flags = _flags(prev.device, flags)
    check("awq_fold_scale", lib.awq_fold_scale(prev.data_ptr(), _DT[prev.dtype], rows, cols,
                                               prev.stride(0) if rows > 1 else cols,
                                               s.data_ptr(), axis, flags.data_ptr(),
                                               _stream(prev)))
    return flags


def pack_int4(W: torch.Tensor, s: torch.Tensor, cfg: AwqConfig = AwqConfig(),
              with_codes: bool = False, flags: torch.Tensor | None = None,
              clip: torch.Tensor | None = None) -> PackResult:
    """Packed codes of Q(W s) (clipped by the per-group ratios `clip`, if given), fp16 group
    steps and fp16 s."""
    lib = _lib.load()
    _dev(W, "W")
    _dev(s, "s")
    N, K = W.shape
    if s.shape != (K,) or s.dtype != torch.float32:
        raise ValueError("s must be fp32 [K]")
    if clip is not None:
        _dev(clip, "clip")
        if clip.shape != (N, K // cfg.group) or clip.dtype != torch.float32:
            raise ValueError("clip must be fp32 [N, K/group]")
    c = cfg.c()
    flags = _flags(W.device, flags)
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    scales16 = torch.empty((N, K // cfg.group), dtype=torch.float16, device=W.device)
    s16 = torch.empty(K, dtype=torch.float16, device=W.device)
    codes = torch.empty((N, K), dtype=torch.int8, device=W.device) if with_codes else None
    zeros = torch.empty((N, K // cfg.group), dtype=torch.uint8, device=W.device) \
        if cfg.zero_point else None
    check("awq_pack_int4", lib.awq_pack_int4(
        W.data_ptr(), _DT[W.dtype], N, K, s.data_ptr(),
        clip.data_ptr() if clip is not None else None, c, qweight.data_ptr(),
        scales16.data_ptr(), zeros.data_ptr() if zeros is not None else None, s16.data_ptr(),
        codes.data_ptr() if codes is not None else None, flags.data_ptr(), _stream(W)))
    return PackResult(qweight, scales16, s16, codes, flags, zeros)


def _w4a16_check(A, qweight, scales16, s16, group, zeros):
    for t, nm in ((A, "A"), (qweight, "qweight"), (scales16, "scales16")):
        _dev(t, nm)
    if s16 is not None:
        _dev(s16, "s16")
    M, K = A.shape
    N = qweight.shape[0]
    if A.dtype != torch.float16 or scales16.dtype != torch.float16 or \
            (s16 is not None and s16.dtype != torch.float16):
        raise ValueError("A, scales16 and s16 must be fp16")
    if qweight.shape != (N, K // 8) or scales16.shape != (N, K // group) or \
            (s16 is not None and s16.shape != (K,)):
        raise ValueError("packed artefact shapes do not match A")
    if zeros is not None:
        _dev(zeros, "zeros")
        if zeros.shape != (N, K // group) or zeros.dtype != torch.uint8:
            raise ValueError("zeros must be uint8 [N, K/group]")
    return M, N, K


def w4a16_gemm(A: torch.Tensor, qweight: torch.Tensor, scales16: torch.Tensor,
               s16: torch.Tensor | None, group: int = 128, out: torch.Tensor | None = None,
               zeros: torch.Tensor | None = None) -> torch.Tensor:
    """Y = (A / s) (c(q) * step)^T, fp16 [M, N], c(q) = q (symmetric) or q - z (zeros given);
    s16 = None when s^-1 is folded into A's producer."""
    lib = _lib.load()
    M, N, K = _w4a16_check(A, qweight, scales16, s16, group, zeros)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    check("w4a16_gemm", lib.w4a16_gemm(A.data_ptr(), M, N, K, group, qweight.data_ptr(),
                                       scales16.data_ptr(),
                                       zeros.data_ptr() if zeros is not None else None,
                                       s16.data_ptr() if s16 is not None else None, out.data_ptr(),
                                       _stream(A)))
    return out


def w4a16_gemm_workspace_bytes(M: int, N: int, K: int, group: int = 128) -> int:
    """Bytes of the w4a16_gemm_ws workspace for these sizes (0: none needed)."""
    return int(_lib.load().w4a16_gemm_workspace_bytes(M, N, K, group))


# w4a16_gemm_ws workspaces kept per (device, stream), so that calls on one stream share one
_W4A16_WS: dict = {}


def w4a16_gemm_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """The cached w4a16_gemm_ws workspace of the current stream on `device`, at least `nbytes`
    bytes (a larger one replaces a smaller one)."""
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _W4A16_WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _W4A16_WS[key] = ws
    return ws


def w4a16_gemm_ws(A: torch.Tensor, qweight: torch.Tensor, scales16: torch.Tensor,
                  s16: torch.Tensor | None, group: int = 128, out: torch.Tensor | None = None,
                  zeros: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """w4a16_gemm with a workspace (K split over workgroups for M <= 64). workspace: a uint8
    device tensor of at least w4a16_gemm_workspace_bytes bytes, or None for the cached one of
    the current stream."""
    lib = _lib.load()
    M, N, K = _w4a16_check(A, qweight, scales16, s16, group, zeros)
    need = w4a16_gemm_workspace_bytes(M, N, K, group)
    if workspace is None:
        workspace = w4a16_gemm_workspace(A.device, need)
    else:
        _dev(workspace, "workspace")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=A.device)
    check("w4a16_gemm_ws", lib.w4a16_gemm_ws(
        A.data_ptr(), M, N, K, group, qweight.data_ptr(), scales16.data_ptr(),
        zeros.data_ptr() if zeros is not None else None,
        s16.data_ptr() if s16 is not None else None, out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream(A)))
    return out
