"""CPU oracle for the AWQ search, INT4 pack and W4A16 path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import or call this module. The GPU library never uses it and shares no code with it.

Plain, slow, step-by-step numpy. Floating-point steps that decide an integer (the scaled weight,
the group step, the quotient that is rounded) are done in IEEE fp32 exactly as specified, because
the integer codes must come out bit-identical on both sides; everything else is fp64.

Pages followed, cited by title and section:
  [notes]   bg51717.github.io/14592 -- notes on the paper "AWQ: Activation-aware Weight
            Quantization for LLM Compression and Acceleration" (arXiv 2306.00978);
            sections 发现 (finding) and 方法 (method) with its equations Q(w), Q(w*s)*x/s,
            the objective L(s) and the grid s = s_X^alpha.
  [eng]     qwbw.cn/news/39982 -- "AWQ 量化方案：激活感知的权重量化与工程实现全解析";
            section 二 (equivalent transform W*X = (W/s)*(X*s)) and section 三 (core algorithm:
            awq_quantize and QuantLinear).
  [schemes] luoboask.github.io/fde-learning/04-inference-optimization/quantization-schemes/ --
            "量化方案详解"; section AWQ (why activation-aware beats uniform, worked example)
            and section GPTQ (layer objective written as a quadratic form in H = X^T X).
  [fa-awq]  ai6s.net/6a17bcfb662f9a54cb77d38b.html -- "FlashAttention与AWQ量化：模型权重怎么压缩
            又不掉精度？"; class AWQQuantizer (bits -> max_val = 2^(bits-1)-1).

Readings taken where the pages are silent, ambiguous or disagree (each is also used below):
  R1  step Delta = max|w s| / (2^(b-1) - 1) ([eng] 三, [fa-awq]); [notes] 方法 prints 2^(b-1).
  R2  codes clamped to [-2^(b-1), 2^(b-1) - 1] ([eng] 三).
  R3  s multiplies W along the input channel and divides X ([notes] 方法); [eng] writes W/s.
  R4  one step per (output row, group of 128 consecutive input channels) (storage shape in [eng] 三).
  R5  s = max(s_X, s_floor)^alpha with s_floor = fp32(1e-5); no normalisation of s.
  R6  alpha_i = i / (n_grid - 1), i = 0..n_grid-1 (both ends of [0, 1], [notes] 方法).
  R7  rounding is round-half-to-even of the fp32-rounded quotient (torch.round in [eng] 三).
  R8  an all-zero group (or a step that underflows to 0) has step 0 and codes 0.
  R9  the loss is reported as the mean of squares ||.||_F^2 / (M N); argmin is unchanged.
  R10 ties in the loss go to the lowest alpha index.
  R11 packing: 8 two's-complement nibbles per uint32, element 8j+t at bits 4t ([eng] 三 says
      "INT4 packed" only); steps and s stored as fp16 (round to nearest even).
  R12 W4A16 divides the activation by s: y = sum_k (A[m,k]/s[k]) q[n,k] step[n,k/G].
  R17 clipping ([notes] 方法 lists "clip the scaled-up weights" among further optimisations and
      says nothing more): per (row, group), W*s is clipped to [-r max|W*s|, r max|W*s|] before
      it is quantized; r is chosen on the grid 1 .. clip_min at the fixed s*, by the part of the
      output error that the group causes on its own (the [notes] objective restricted to the
      group's channels, so that the choices are separable), lowest index on ties.
  R19 zero point ("AWQ 量化方案..." 三 Step 4 names a scale and a zero point per group; the
      worked example of "量化方案详解", section AWQ, spreads 2^4 levels over a group's range
      [min, max]): Delta = (max - min) / (2^b - 1), z = rint(-min / Delta), unsigned codes
      clamp(rint(w s / Delta) + z, 0, 2^b - 1), each step in IEEE fp32, one rounding per step.
  R18 folding ([notes] 方法, further optimisations: fuse the input's down-scaling into the
      previous operator): every weight that reads the same X shares one s, searched on the
      row-concatenated weights; s^-1 is folded into the previous operator's parameters along
      its output channels (fp32 division, one rounding to their dtype), after which the
      quantized layer takes its input unscaled (W4A16 without the division by s).
"""
from __future__ import annotations

import math
import numpy as np

F32 = np.float32
F64 = np.float64


# ---------------------------------------------------------------------------------------------
# Activation statistics
# ---------------------------------------------------------------------------------------------
def act_stats(X: np.ndarray, chunk_rows: int = 4096) -> np.ndarray:
    """s_X[k] = mean over tokens m of |X[m, k]|  ([notes] 方法: s_X from the input; [eng] 三
    Step 1 act_norm = |X| averaged over samples).

    The column sum is accumulated in fp64 and divided by M in fp64, then rounded once to fp32.
    For fp16 X every |x| is a multiple of 2^-24 and the sum stays exact (hence independent of
    the order) while it is below 2^29.
    """
    X = np.asarray(X)
    if not np.all(np.isfinite(X)):
        raise ValueError("non-finite activation")
    M, K = X.shape
    S = np.zeros(K, dtype=F64)
    for r0 in range(0, M, chunk_rows):
        S += np.abs(X[r0:r0 + chunk_rows].astype(F64)).sum(axis=0)
    return (S / F64(M)).astype(F32)


# ---------------------------------------------------------------------------------------------
# Grid of scales
# ---------------------------------------------------------------------------------------------
def alpha_grid(n_grid: int) -> list[float]:
    """alpha_i = i/(n_grid-1) as fp64 quotients (R6; [notes] 方法: alpha searched in [0, 1])."""
    if n_grid < 2:
        raise ValueError("n_grid must be >= 2")
    return [i / (n_grid - 1) for i in range(n_grid)]


def scale_table(sx: np.ndarray, n_grid: int, s_floor: float = 1e-5) -> np.ndarray:
    """s_i[k] = fp32( max(s_X[k], s_floor)^alpha_i )  ([notes] 方法: s = s_X^alpha; R5).

    The floor is compared in fp32; the power is the fp64 libm pow of the fp64 operands, then
    rounded to fp32.
    """
    base = np.maximum(np.asarray(sx, dtype=F32), F32(s_floor))
    out = np.empty((n_grid, base.shape[0]), dtype=F32)
    for i, a in enumerate(alpha_grid(n_grid)):
        out[i] = np.array([math.pow(float(b), a) for b in base], dtype=F64).astype(F32)
    return out


# ---------------------------------------------------------------------------------------------
# Group-wise symmetric quantization of W * s
# ---------------------------------------------------------------------------------------------
def code_range(bits: int) -> tuple[int, int]:
    """(qmin, qmax) = (-2^(b-1), 2^(b-1)-1)  (R1, R2; [fa-awq] max_val, [eng] 三 clamp)."""
    return -(2 ** (bits - 1)), 2 ** (bits - 1) - 1


def quantize_zp(W: np.ndarray, s: np.ndarray, bits: int = 4, group: int = 128, clip=None):
    """Zero-point (asymmetric) codes of Q(W*s), one step and one zero point per (row, group)
    (R19; "量化方案详解", section AWQ, worked example: a range [-3.2, 3.2] on 2^4 levels has the step
    6.4 / 15 = 0.427; "AWQ 量化方案..." 三 Step 4 names a scale and a zero point per group):
      ws    = fp32(w * s[k])                            (clipped first, as in `quantize`)
      Delta = fp32( fp32(max ws - min ws) / (2^b - 1) )  over the group
      z     = clamp(rint(fp32(-min ws / Delta)), 0, 2^b - 1)
      q     = clamp(rint(fp32(ws / Delta)) + z, 0, 2^b - 1)
    and Q(w*s) = (q - z) * Delta. A group with Delta = 0 gets q = z = 0 (R8).
    Returns (q uint8 [N, K], Delta fp32 [N, K/group], z uint8 [N, K/group])."""
    W = np.asarray(W)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmax_u = 2 ** bits - 1
    ws = W.astype(F32) * np.asarray(s, dtype=F32)[None, :]
    wsg = ws.reshape(N, K // group, group)
    if clip is not None:
        r = np.asarray(clip, dtype=F32).reshape(N, K // group)
        if not np.all((r > 0) & (r <= 1)):
            raise ValueError("clip ratios must lie in (0, 1]")
        c = (r * np.abs(wsg).max(axis=2)).astype(F32)
        wsg = np.clip(wsg, -c[:, :, None], c[:, :, None])
    mx = wsg.max(axis=2)
    mn = wsg.min(axis=2)
    rng_ = (mx - mn).astype(F32)                               # fp32 - fp32 -> fp32
    delta = (rng_ / F32(qmax_u)).astype(F32)
    live = delta > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        z = np.where(live, np.clip(np.rint((-mn / delta).astype(F32)), 0, qmax_u), F32(0))
        t = (wsg / delta[:, :, None]).astype(F32)
    q = np.where(live[:, :, None], np.clip(np.rint(t) + z[:, :, None], 0, qmax_u), F32(0))
    return q.reshape(N, K).astype(np.uint8), delta, z.astype(np.uint8)


def quantize(W: np.ndarray, s: np.ndarray, bits: int = 4, group: int = 128, clip=None):
    """Codes and steps of Q(W*s), one step per (row, group of `group` input channels).

    Steps in the order of [notes] 方法 (Q(w) = Delta * Round(w / Delta)) and [eng] 三 Step 4:
      ws    = fp32(w * s[k])                        the scaled weight (R3)
      m     = max |ws| over the group               (R4)
      Delta = fp32(m / qmax)                        IEEE division (R1)
      q     = clamp(rint(fp32(ws / Delta)))         round half to even (R7), clamp (R2)
    With `clip` (fp32 ratios r in (0, 1], one per (row, group)), the scaled weights are first
    clipped to [-c, c], c = fp32(r * m) ([notes] 方法, further optimisations: clip the scaled-up
    weights; R17), and the steps above run on the clipped values (so m becomes c).
    Returns (q int8 [N, K], Delta fp32 [N, K/group]).
    """
    W = np.asarray(W)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmin, qmax = code_range(bits)
    w = W.astype(F32)                                  # exact for fp16 / fp32 inputs
    ws = w * np.asarray(s, dtype=F32)[None, :]         # fp32 * fp32 -> fp32, round to nearest
    wsg = ws.reshape(N, K // group, group)
    if clip is not None:
        r = np.asarray(clip, dtype=F32).reshape(N, K // group)
        if not np.all((r > 0) & (r <= 1)):
            raise ValueError("clip ratios must lie in (0, 1]")
        c = (r * np.abs(wsg).max(axis=2)).astype(F32)  # fp32 * fp32 -> fp32
        wsg = np.clip(wsg, -c[:, :, None], c[:, :, None])
    m = np.abs(wsg).max(axis=2)
    delta = (m / F32(qmax)).astype(F32)                # fp32 / fp32 -> fp32
    live = delta > 0                                   # R8
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (wsg / delta[:, :, None]).astype(F32)      # fp32 / fp32 -> fp32
    q = np.where(live[:, :, None], np.clip(np.rint(t), qmin, qmax), F32(0))
    return q.reshape(N, K).astype(np.int8), delta


def dequant_scaled(q: np.ndarray, delta: np.ndarray, group: int = 128, z=None) -> np.ndarray:
    """Q(W*s) = q * Delta (or (q - z) * Delta with zero points), in fp64, shape [N, K]."""
    qq = q.astype(F64)
    if z is not None:
        qq = qq - np.repeat(np.asarray(z).astype(F64), group, axis=1)
    return qq * np.repeat(delta.astype(F64), group, axis=1)


def error_matrix(W: np.ndarray, q: np.ndarray, delta: np.ndarray, s: np.ndarray,
                 group: int = 128, z=None) -> np.ndarray:
    """E = Q(W*s) / s - W in fp64. X @ E^T is Q(W*s)(s^-1 X) - W X in the tokens-by-rows
    layout, by linearity ([notes] 方法 objective; [eng] 二 equivalent transform)."""
    return dequant_scaled(q, delta, group, z) / np.asarray(s, dtype=F64)[None, :] - \
        np.asarray(W).astype(F64)


# ---------------------------------------------------------------------------------------------
# Loss
# ---------------------------------------------------------------------------------------------
def output_loss(X: np.ndarray, W: np.ndarray, s: np.ndarray, QWs: np.ndarray) -> float:
    """L = || Q(W s)(s^-1 X) - W X ||_F^2 / (M N), written literally in fp64
    ([notes] 方法 objective; R9). X is [M, K] (tokens x input channels), W and QWs = Q(W s) are
    [N, K]; the scaled activation is X / s and the outputs are compared as [M, N] matrices."""
    X64 = np.asarray(X).astype(F64)
    Yq = (X64 / np.asarray(s, dtype=F64)[None, :]) @ np.asarray(QWs, dtype=F64).T
    Y = X64 @ np.asarray(W).astype(F64).T
    D = Yq - Y
    return float((D * D).sum() / (X64.shape[0] * D.shape[1]))


def gram(X: np.ndarray, chunk_rows: int = 4096) -> np.ndarray:
    """H = X^T X in fp64 ([schemes] GPTQ: the layer objective as a quadratic form in H)."""
    X = np.asarray(X)
    K = X.shape[1]
    H = np.zeros((K, K), dtype=F64)
    for r0 in range(0, X.shape[0], chunk_rows):
        c = X[r0:r0 + chunk_rows].astype(F64)
        H += c.T @ c
    return H


def loss_gram(H: np.ndarray, E: np.ndarray, M: int) -> float:
    """L = sum_n E_n H E_n^T / (M N): the same value as output_loss, since
    ||X E^T||_F^2 = trace(E X^T X E^T)."""
    return float(((E @ H) * E).sum() / (M * E.shape[0]))


def clip_grid(n_clip: int = 11, clip_min: float = 0.5) -> np.ndarray:
    """Clip ratios r_j = fp32(1 - (1 - clip_min) j / (n_clip - 1)), j = 0 .. n_clip-1: from no
    clipping (r = 1) down to clip_min, evenly in fp64 (clip_min taken as an fp32 value, the
    precision of the configuration), each rounded once to fp32 (R17)."""
    cm = float(F32(clip_min))
    if n_clip < 2 or not (0.0 < cm < 1.0):
        raise ValueError("n_clip >= 2 and 0 < clip_min < 1 required")
    return np.array([1.0 - (1.0 - cm) * j / (n_clip - 1) for j in range(n_clip)],
                    dtype=F64).astype(F32)


def group_errors(E: np.ndarray, group: int = 128, X=None, H=None) -> np.ndarray:
    """err[n, g] = sum_m ( sum_{k in g} X[m, k] E[n, k] )^2: the part of the output error of row
    n that the channels of group g cause on their own, in fp64. With H = X^T X it is the same
    value as E_g H_gg E_g^T (the diagonal block of H)."""
    E = np.asarray(E, dtype=F64)
    N, K = E.shape
    out = np.empty((N, K // group), dtype=F64)
    for g in range(K // group):
        sl = slice(g * group, (g + 1) * group)
        if H is not None:
            Eg = E[:, sl]
            out[:, g] = np.einsum("nk,kl,nl->n", Eg, np.asarray(H, dtype=F64)[sl, sl], Eg)
        else:
            P = np.asarray(X).astype(F64)[:, sl] @ E[:, sl].T          # [M, N]
            out[:, g] = (P * P).sum(axis=0)
    return out


def clip_search(W, X, s, bits: int = 4, group: int = 128, n_clip: int = 11,
                clip_min: float = 0.5, H=None, zero_point: bool = False):
    """Per (row, group), the clip ratio of `clip_grid` whose quantization of W*s gives the
    smallest group error (`group_errors`), the lowest index on ties (R17, R10). The search runs
    at a fixed s (typically s*). Returns {"ratio": fp32 [N, K/group], "best": int [N, K/group],
    "err": fp64 [n_clip, N, K/group]}."""
    r = clip_grid(n_clip, clip_min)
    W = np.asarray(W)
    N, K = W.shape
    s = np.asarray(s, dtype=F32)
    err = np.empty((n_clip, N, K // group), dtype=F64)
    for j in range(n_clip):
        full = np.full((N, K // group), r[j], dtype=F32)
        if zero_point:
            q, d, z = quantize_zp(W, s, bits, group, clip=full)
        else:
            (q, d), z = quantize(W, s, bits, group, clip=full), None
        E = error_matrix(W, q, d, s, group, z)
        err[j] = group_errors(E, group, X=None if H is not None else X, H=H)
    best = np.zeros((N, K // group), dtype=np.int64)
    for j in range(1, n_clip):                      # strict < keeps the lowest index on ties
        better = err[j] < err[best, np.arange(N)[:, None], np.arange(K // group)[None, :]]
        best = np.where(better, j, best)
    return {"ratio": r[best], "best": best, "err": err}


def argmin_lowest(losses) -> int:
    """Smallest index attaining the minimum (R10; [notes] 方法 alpha* = argmin L)."""
    best = 0
    for i in range(1, len(losses)):
        if losses[i] < losses[best]:
            best = i
    return best


def search_layer(W, X, sx, bits: int = 4, group: int = 128, n_grid: int = 20,
                 s_floor: float = 1e-5, form: str = "direct", H=None, zero_point: bool = False):
    """Grid search of [notes] 方法: for each alpha_i, s_i = s_X^alpha_i, quantize W*s_i, score
    L(s_i); alpha* = argmin. form='direct' evaluates the literal objective, form='gram' the
    identical quadratic form with H = X^T X (computed here unless given)."""
    S = scale_table(sx, n_grid, s_floor)
    M = np.asarray(X).shape[0]
    if form == "gram" and H is None:
        H = gram(X)
    losses = np.empty(n_grid, dtype=F64)
    for i in range(n_grid):
        if zero_point:
            q, delta, z = quantize_zp(W, S[i], bits, group)
        else:
            (q, delta), z = quantize(W, S[i], bits, group), None
        if form == "direct":
            losses[i] = output_loss(X, W, S[i], dequant_scaled(q, delta, group, z))
        elif form == "gram":
            losses[i] = loss_gram(H, error_matrix(W, q, delta, S[i], group, z), M)
        else:
            raise ValueError(form)
    best = argmin_lowest(losses)
    return {"losses": losses, "best": best, "alpha": alpha_grid(n_grid)[best],
            "s_best": S[best].copy(), "scales": S}


def search_shared(Ws, X, sx, bits: int = 4, group: int = 128, n_grid: int = 20,
                  s_floor: float = 1e-5, form: str = "direct", H=None, zero_point: bool = False):
    """One alpha for several weights that read the same input X (q/k/v, gate/up): the search of
    `search_layer` on the row-concatenated weights [W_0; W_1; ...] ([notes] 方法: the scale
    multiplies input channels and its inverse is folded into the previous operator, so every
    consumer of that operator's output must use the same s; R18). The loss is the mean of
    squares over all N_0 + N_1 + ... outputs."""
    Wc = np.concatenate([np.asarray(W) for W in Ws], axis=0)
    return search_layer(Wc, X, sx, bits, group, n_grid, s_floor, form, H, zero_point)


def fold_scale(prev: np.ndarray, s: np.ndarray, axis: int) -> np.ndarray:
    """The previous operator's parameters with s^-1 folded in ([notes] 方法, further
    optimisations: fuse the input's down-scaling into the previous operator; R18): along `axis`
    (1: columns, e.g. a norm weight [1, K]; 0: rows, e.g. the output channels of a previous
    linear layer [K, ...]) every entry is divided by s of its channel, fp32(fp32(p) / s), then
    rounded once to prev's dtype."""
    p = np.asarray(prev)
    s = np.asarray(s, dtype=F32)
    s_b = s[None, :] if axis == 1 else s[:, None]
    return (p.astype(F32) / s_b).astype(F32).astype(p.dtype)


def relative_gap(losses) -> float:
    """(runner-up - best) / best: how clearly the grid point is the minimum."""
    ls = np.sort(np.asarray(losses, dtype=F64))
    return float((ls[1] - ls[0]) / ls[0]) if ls[0] > 0 else float("inf")


# ---------------------------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------------------------
def pack_int4(q: np.ndarray) -> np.ndarray:
    """qweight[n, j] = sum_t (q[n, 8j+t] & 0xF) << 4t  (R11)."""
    q = np.asarray(q)
    N, K = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    nib = (q.astype(np.int64) & 0xF).astype(np.uint64)
    out = np.zeros((N, K // 8), dtype=np.uint64)
    for t in range(8):
        out |= nib[:, t::8] << np.uint64(4 * t)
    return out.astype(np.uint32)


def unpack_uint4(qweight: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 for zero-point codes: unsigned nibbles 0..15, uint8 [N, 8 * cols]."""
    qw = np.asarray(qweight).astype(np.uint64)
    N, C = qw.shape
    out = np.empty((N, 8 * C), dtype=np.uint8)
    for t in range(8):
        out[:, t::8] = ((qw >> np.uint64(4 * t)) & np.uint64(0xF)).astype(np.uint8)
    return out


def unpack_int4(qweight: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: sign-extended nibbles, int8 [N, 8 * cols]."""
    qw = np.asarray(qweight).astype(np.uint64)
    N, C = qw.shape
    out = np.empty((N, 8 * C), dtype=np.int8)
    for t in range(8):
        nib = ((qw >> np.uint64(4 * t)) & np.uint64(0xF)).astype(np.int64)
        out[:, t::8] = np.where(nib >= 8, nib - 16, nib)
    return out


def pack_layer(W, s, bits: int = 4, group: int = 128, clip=None, zero_point: bool = False):
    """The stored result of [eng] 三 (QuantLinear(q_weight, scales_per_group, awq_scale)):
    packed codes of Q(W*s), per-group fp16 steps and the per-channel s in fp16 (R11); with zero
    points (R19) the codes are the unsigned 0 .. 2^b-1 of `quantize_zp` in the same nibble
    layout and "zeros" holds z per (row, group) as uint8. The codes are those of the quantizer
    (with the clip ratios, if given), not re-derived from the fp16 step."""
    if zero_point:
        q, delta, z = quantize_zp(W, s, bits, group, clip=clip)
    else:
        (q, delta), z = quantize(W, s, bits, group, clip=clip), None
    return {"qweight": pack_int4(q), "scales16": delta.astype(np.float16),
            "s16": np.asarray(s, dtype=F32).astype(np.float16), "codes": q, "delta": delta,
            "zeros": z}


# ---------------------------------------------------------------------------------------------
# W4A16
# ---------------------------------------------------------------------------------------------
def w4a16(A: np.ndarray, qweight: np.ndarray, scales16: np.ndarray, s16,
          group: int = 128, zeros=None) -> np.ndarray:
    """Y = (A / s) @ (q * step)^T in fp64 from the packed artefacts ([eng] 三 QuantLinear.forward:
    scale the input per channel, dequantize qweight * scales repeated over each group, then a
    linear layer; R12: the activation is divided by s because W was multiplied by s). With
    s16 = None the division has been folded into the producer of A (R18): Y = A @ (q step)^T.
    With zero points (R19) the codes are unsigned and the weight is (q - z) * step."""
    if zeros is None:
        q = unpack_int4(qweight).astype(F64)
    else:
        q = unpack_uint4(qweight).astype(F64) - np.repeat(np.asarray(zeros).astype(F64), group,
                                                          axis=1)
    Wd = q * np.repeat(np.asarray(scales16).astype(F64), group, axis=1)
    Ap = np.asarray(A).astype(F64)
    if s16 is not None:
        Ap = Ap / np.asarray(s16).astype(F64)[None, :]
    return Ap @ Wd.T


def accuracy_report(y_test: np.ndarray, y_ref: np.ndarray) -> dict:
    """Max abs, max rel (|ref| clamped at 1e-6), mean abs errors and the relative Frobenius
    error (metric definitions of "FlashAttention的量化：INT8和FP8怎么用才不影响精度？",
    cyqw.cn/news/1226870, section 精度验证)."""
    t = np.asarray(y_test, dtype=F64)
    r = np.asarray(y_ref, dtype=F64)
    d = np.abs(t - r)
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "max_rel": float((d / np.maximum(np.abs(r), 1e-6)).max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "rel_fro": float(np.linalg.norm(t - r) / max(np.linalg.norm(r), 1e-300))}
