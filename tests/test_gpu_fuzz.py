"""Seeded random configurations through the whole path against the oracle: shapes (ragged N, K
a multiple of the group, token counts from 1 up), dtypes of W and X, 3 and 4 bits, groups of 64
and 128, symmetric and zero-point codes, both search forms. The configurations are drawn once
from a fixed seed, so the list is the same on every run.

Every other configuration goes through awq_stats_search_layer (s_X and the search in one call;
in the Gram form with fp16 X the column sums come from the transpose pass), the rest through
awq_act_stats then awq_search_layer.

Per configuration: s_X bit-exact; every per-alpha loss within 1e-4 relative of the oracle's
(layers with fewer than 256 rows or tokens take the fp32 contraction); alpha* equal to the
oracle's unless the oracle's two best losses are within twice that bar; at the GPU's alpha*,
codes, packed words, fp16 steps and zero points bit-exact; W4A16 on the packed result within 2e-3 of the oracle's
(when K is a multiple of 128, which W4A16 needs with groups of 64).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import exact_ref as ex

pytestmark = pytest.mark.gpu
FLAG_STATS_INEXACT = 1 << 2

def _configs(count=24, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for c in range(count):
        group = int(g.choice([64, 128]))
        k = int(g.integers(2, 10)) * 128 if group == 128 else int(g.integers(2, 19)) * 64
        n = int(g.choice([int(g.integers(1, 64)), int(g.integers(64, 700))]))
        m = int(g.choice([int(g.integers(1, 40)), int(g.integers(40, 1500))]))
        out.append(dict(
            id=f"c{c}_n{n}_k{k}_m{m}", n=n, k=k, m=m, group=group,
            bits=int(g.choice([3, 4])), zp=bool(g.integers(0, 2)),
            form=str(g.choice(["direct", "gram"])),
            wdt=[np.float16, np.float32][int(g.integers(0, 2))],
            xdt=["f16", "bf16", "f32"][int(g.integers(0, 3))],
            outliers=int(g.integers(0, 6)), seed=int(g.integers(0, 2**31)), fused=c % 2 == 1))
    return out


CONFIGS = _configs()


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import post_weight_quantization_channel_amd as m
    from post_weight_quantization_channel_amd import _lib
    _lib.load()
    return m


def _inputs(cfg):
    g = np.random.default_rng(cfg["seed"])
    W = (0.02 * g.standard_normal((cfg["n"], cfg["k"]))).astype(cfg["wdt"])
    gains = np.exp(g.standard_normal(cfg["k"]))
    if cfg["outliers"]:
        gains[g.choice(cfg["k"], cfg["outliers"], replace=False)] *= 30.0
    X64 = g.standard_normal((cfg["m"], cfg["k"])) * gains[None, :]
    if cfg["xdt"] == "f16":
        return W, X64.astype(np.float16), torch.float16
    if cfg["xdt"] == "f32":
        return W, X64.astype(np.float32), torch.float32
    # bf16: round to nearest even in fp32 bits; the oracle reads the same values as fp32
    x32 = X64.astype(np.float32)
    b = x32.view(np.uint32)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return W, b.view(np.float32), torch.bfloat16


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c["id"] for c in CONFIGS])
def test_fuzz_path_against_oracle(awq, cfg):
    W, X, tdt = _inputs(cfg)
    print("  ", cfg, flush=True)
    Wt = torch.from_numpy(W).cuda()
    Xt = torch.from_numpy(X).cuda().to(tdt)
    acfg = awq.AwqConfig(bits=cfg["bits"], group=cfg["group"], form=cfg["form"],
                         zero_point=cfg["zp"])
    if cfg["fused"]:
        sx, res = awq.stats_search_layer(Wt, Xt, acfg)
        flags = res.flags
    else:
        sx, flags = awq.act_stats(Xt)
        res = awq.search_layer(Wt, Xt, sx, acfg, flags=flags)
    bg = int(res.best.item())
    p = awq.pack_int4(Wt, res.s_best, acfg, flags=flags, with_codes=True)
    # W4A16 walks K in 128-channel steps: with groups of 64 it needs K % 128 == 0
    run_w4 = cfg["k"] % 128 == 0
    A = np.random.default_rng(cfg["seed"] + 1).standard_normal((5, cfg["k"])).astype(np.float16)
    if run_w4:
        Y = awq.w4a16_gemm(torch.from_numpy(A).cuda(), p.qweight, p.scales16, p.s16,
                           group=cfg["group"], zeros=p.zeros)
    torch.cuda.synchronize()
    # bf16 / fp32 column sums that may round in fp64 are flagged (then s_X is the sum in this
    # library's order; it still matches the oracle's here)
    bits = {"f16": None, "bf16": 7, "f32": 23}[cfg["xdt"]]
    may_round = bits is not None and ex.stats_sum_may_round(X, bits)
    assert int(flags.item()) == (FLAG_STATS_INEXACT if may_round else 0)

    sx_o = oracle.act_stats(X)
    assert np.array_equal(sx.cpu().numpy(), sx_o)
    form = "gram" if 2 * cfg["m"] > cfg["k"] else "direct"
    orc = oracle.search_layer(W, X, sx_o, bits=cfg["bits"], group=cfg["group"], form=form,
                              zero_point=cfg["zp"])
    tol = 1e-4
    lg = res.losses.cpu().numpy()
    live = orc["losses"] > 0
    rel = np.abs(lg - orc["losses"])[live] / orc["losses"][live]
    assert rel.size == 0 or rel.max() <= tol, f"loss rel err {rel.max():.3e}"
    assert np.all(lg[~live] == 0.0)
    if oracle.relative_gap(orc["losses"]) > 2 * tol:
        assert bg == orc["best"], (bg, orc["best"])
    else:
        assert orc["losses"][bg] <= orc["losses"].min() * (1 + 2 * tol) + 1e-300
    o = oracle.pack_layer(W, orc["scales"][bg], bits=cfg["bits"], group=cfg["group"],
                          zero_point=cfg["zp"])
    assert np.array_equal(p.codes.cpu().numpy(), o["codes"])
    assert np.array_equal(p.qweight.cpu().numpy().view(np.uint32), o["qweight"])
    assert np.array_equal(p.scales16.cpu().numpy().view(np.uint16),
                          o["scales16"].view(np.uint16))
    if cfg["zp"]:
        assert np.array_equal(p.zeros.cpu().numpy(), o["zeros"])
    if run_w4:
        ref = oracle.w4a16(A, o["qweight"], o["scales16"], o["s16"], group=cfg["group"],
                           zeros=o["zeros"])
        assert oracle.accuracy_report(Y.cpu().numpy(), ref)["rel_fro"] <= 2e-3
