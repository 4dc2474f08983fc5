"""Seeded synthetic inputs for the AWQ layer workloads.

This module only draws random tensors; it holds none of the quantization method's arithmetic.
Both the GPU library's callers (tests, bench) and the CPU oracle take their inputs from here.

The shapes and value distributions stand in for the LLaMA-7B / 70B-class calibration workloads
that the pages describe (128 calibration samples of 512 tokens, hidden size 4096, MLP 11008,
group 128): no public dataset or trained weight is used.

Recipe (all draws in float64 from numpy's PCG64, rounded to the layer dtype on the host):
  * seed = 1000 * config + t + 10 * j, with t = 0 for W, 1 for the base X, 2 for the channel
    magnitudes / outlier choice, 3 for W4A16 activations, and j the index of a weight within a
    config;
  * W = 0.02 * N(0, 1);
  * X is drawn in 4096-row chunks from one stream.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CHUNK_ROWS = 4096


def rng(config: int, t: int, j: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config + t + 10 * j))


def _cast(a64: np.ndarray, dtype) -> np.ndarray:
    return a64.astype(dtype)


def weight(config: int, n: int, k: int, dtype=np.float16, j: int = 0) -> np.ndarray:
    """W = 0.02 * N(0,1), shape [n, k] (out_features, in_features)."""
    return _cast(0.02 * rng(config, 0, j).standard_normal((n, k)), dtype)


def channel_gains_lognormal(config: int, k: int, outlier_frac: float, outlier_mult: float,
                            j: int = 0) -> np.ndarray:
    """Per-channel magnitudes c_k ~ lognormal(0, 1); the round(frac*k) largest are multiplied."""
    c = rng(config, 2, j).lognormal(0.0, 1.0, size=k)
    n_out = int(round(outlier_frac * k))
    if n_out:
        idx = np.argsort(c, kind="stable")[-n_out:]
        c[idx] *= outlier_mult
    return c


def channel_gains_choice(config: int, k: int, n_out: int, outlier_mult: float,
                         j: int = 0) -> np.ndarray:
    """Unit magnitudes with n_out channels picked by rng.choice (no replacement) multiplied."""
    c = np.ones(k)
    idx = rng(config, 2, j).choice(k, n_out, replace=False)
    c[idx] *= outlier_mult
    return c


def activations(config: int, m: int, gains: np.ndarray, dtype=np.float16, j: int = 0,
                absolute: bool = False) -> np.ndarray:
    """X[m, k] = N(0,1) * gains[k] (or |N(0,1)| * gains[k]), drawn in 4096-row chunks."""
    k = gains.shape[0]
    g = rng(config, 1, j)
    out = np.empty((m, k), dtype=dtype)
    for r0 in range(0, m, CHUNK_ROWS):
        r1 = min(m, r0 + CHUNK_ROWS)
        z = g.standard_normal((r1 - r0, k))
        if absolute:
            np.abs(z, out=z)
        z *= gains[None, :]
        out[r0:r1] = z.astype(dtype)
    return out


def correlated_activations(m: int, k: int, rank: int, config: int, dtype=np.float16,
                           noise: float = 0.1) -> np.ndarray:
    """Channels that move together: X = (Z F + noise * N) * gains with Z [m, rank] and
    F [rank, k] standard normal (t = 1 for Z and N, t = 2 for F and the gains), so many channel
    pairs have correlations near +-1. Stands in for the correlated hidden states of a real
    model; the main workloads keep independent channels."""
    g = rng(config, 1)
    gf = rng(config, 2)
    F = gf.standard_normal((rank, k)) / np.sqrt(rank)
    gains = np.exp(gf.standard_normal(k))
    z = g.standard_normal((m, rank)) @ F + noise * g.standard_normal((m, k))
    return (z * gains[None, :]).astype(dtype)


@dataclasses.dataclass
class Layer:
    name: str
    W: np.ndarray          # [N, K]
    X: np.ndarray          # [M, K]
    bits: int = 4
    group: int = 128
    n_grid: int = 20


def c1_layer() -> Layer:
    """512x512 fp32 layer, 256 fp32 tokens, 5 rng.choice channels x20."""
    W = weight(1, 512, 512, np.float32)
    X = activations(1, 256, channel_gains_choice(1, 512, 5, 20.0), np.float32)
    return Layer("c1_512x512_m256_fp32", W, X)


def c2_like_layer(n: int = 4096, k: int = 4096, m: int = 65536, config: int = 2,
                  dtype=np.float16, bits: int = 4) -> Layer:
    """LLaMA-7B attention-projection recipe: lognormal channel gains, top 1% x50."""
    W = weight(config, n, k, dtype)
    X = activations(config, m, channel_gains_lognormal(config, k, 0.01, 50.0), dtype)
    return Layer(f"c{config}_{n}x{k}_m{m}", W, X, bits=bits)


def c3_layers(m: int = 65536, hidden: int = 4096, inter: int = 11008):
    """MLP trio: gate/up [inter, hidden] sharing a C2-style X; down [hidden, inter] with
    X_d = |N(0,1)| and round(0.01*inter) rng.choice channels x30."""
    X = activations(3, m, channel_gains_lognormal(3, hidden, 0.01, 50.0), np.float16)
    gate = weight(3, inter, hidden, np.float16, j=0)
    up = weight(3, inter, hidden, np.float16, j=1)
    n_out = int(round(0.01 * inter))
    Xd = activations(3, m, channel_gains_choice(3, inter, n_out, 30.0, j=2), np.float16, j=2,
                     absolute=True)
    down = weight(3, hidden, inter, np.float16, j=2)
    return [Layer("c3_gate", gate, X), Layer("c3_up", up, X), Layer("c3_down", down, Xd)]


def c5_x(m: int = 65536, k: int = 8192) -> np.ndarray:
    """70B-class activations: N(0,1) with round(0.01*k) rng.choice channels x50."""
    return activations(5, m, channel_gains_choice(5, k, int(round(0.01 * k)), 50.0), np.float16)


def c5_weight(n: int, k: int = 8192, j: int = 0) -> np.ndarray:
    return weight(5, n, k, np.float16, j=j)


def w4a16_random_artifacts(n: int, k: int, group: int = 128, config: int = 4, j: int = 0):
    """Bandwidth-run artefacts: codes U[-8,7], group steps 0.01*|N|, channel scales 1+|N|.

    Codes uniform on the 16 four-bit values are exactly uniformly random 32-bit words (eight
    nibbles each), so the packed words are drawn directly.
    Returns (qweight uint32 [n, k/8], steps fp16 [n, k/group], s fp16 [k]).
    """
    g = rng(config, 0, j)
    qweight = g.integers(0, 2**32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    steps = (0.01 * np.abs(g.standard_normal((n, k // group)))).astype(np.float16)
    s = (1.0 + np.abs(g.standard_normal(k))).astype(np.float16)
    return qweight, steps, s


def w4a16_random_zeros(n: int, k: int, group: int = 128, config: int = 4, j: int = 0):
    """Zero points for zero-point artefacts: uint8 [n, k/group] uniform in 0..15 (t = 2)."""
    return rng(config, 2, j).integers(0, 16, size=(n, k // group)).astype(np.uint8)


def w4a16_activations(m: int, k: int, config: int = 4, j: int = 0) -> np.ndarray:
    """A = N(0,1) fp16 [m, k]."""
    return rng(config, 3, j).standard_normal((m, k)).astype(np.float16)
