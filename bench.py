#!/usr/bin/env python3
"""Benchmark of the AWQ hot path on one MI355X.

One step = one pass of the whole path over the LLaMA-7B-shaped attention projection (W fp16
4096x4096, 65536 calibration tokens = 128 samples x 512 tokens, INT4, group 128, 20 alpha points):
    awq_stats_search_layer (s_X, then the alpha search) -> awq_pack_int4(s*) -> w4a16_gemm
    (decode, M = 1).
The search runs in the Gram form (H = X^T X once, then one K x K contraction per grid point),
and s_X comes out of the pass that transposes X for it (awq_act_stats alone is timed as context);
--form direct times the direct form (X contracted with every error matrix) instead. Inputs are
synthetic (seeded, see workloads/) and resident in HBM before the timed region.

Prints ONE JSON line. `value` is milliseconds per layer (lower is better). Besides the contract
fields it carries
  roofline      the step's longest kernel against the dense fp16 MFMA peak, its duration
                measured with HIP events on the library's stream (in extra steps after the
                timed ones, whose search call waits for its events); `mfma` lists every MFMA
                kernel of the step the same way;
  stages_ms     mean duration of every kernel of the search (the same extra steps);
  other_form    the search in the other form (a few repetitions): ms and its loss kernel;
  clip_search   the clipping search at s* (11 ratios 1 .. 0.5) and the clipped pack: ms; and
                the same search on the operand the step's Gram-form search left in its
                workspace (awq_clip_search_gram);
  shared_qkv    one alpha for three 4096x4096 weights reading the same X (s_X taken in the same
                call), and the fold of s^-1 into the producing norm weight: ms;
  quant_variants  groups of 64 and zero-point codes (and both): the search (ms, its quantize
                and loss kernels), the pack, and W4A16 at M = 1 and 512 on 4096x4096;
  hbm_stages    the bandwidth-bound kernels: algorithmic bytes, GB/s, fraction of 8 TB/s;
  w4a16         the W4A16 kernel at the batch sizes 1, 4, 16, 64, 512 for 4096x4096 and
                11008x4096, over rotated weight copies (> 256 MB, so HBM and not the
                Infinity Cache is measured), replayed from a HIP graph (GPU time per call;
                `us_eager`: the same calls issued one by one from Python): GB/s and fraction
                of 8 TB/s (TFLOP/s and MFMA fraction at M = 512);
  cpu_baseline  the CPU oracle on a bounded sample of the same layer, scaled to ms per layer.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
N_, K_, M_ = 4096, 4096, 65536
N_GRID = 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-w4a16-sweep", action="store_true")
    ap.add_argument("--form", choices=("gram", "direct"), default="gram",
                    help="loss form of the timed search (the other form is reported as context)")
    ap.add_argument("--other-form-reps", type=int, default=3,
                    help="repetitions of the search in the other form (0: skip)")
    ap.add_argument("--clip-reps", type=int, default=5,
                    help="repetitions of the clipping search at s* (0: skip)")
    ap.add_argument("--variant-reps", type=int, default=2,
                    help="repetitions of the zero-point / group-64 search, pack and W4A16")
    ap.add_argument("--shared-reps", type=int, default=3,
                    help="repetitions of the shared q/k/v search and the fold (0: skip)")
    ap.add_argument("--mode", choices=("bench", "traffic"), default="bench",
                    help="traffic: one 1 GiB device copy (counter calibration) and one pass of "
                         "the path in each form, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "search_c2_traffic.json")
CSRC = os.path.join(ROOT, "post_weight_quantization_channel_amd", "csrc")
# the sources each MFMA kernel is compiled from (a counter record is valid only for these bytes)
KERNEL_SOURCES = {
    "lossgemm_kernel": ("lossgemm.hip", "mfma_kloop.h", "device_common.h"),
    "gram_loss_kernel": ("gram.hip", "mfma_kloop.h", "device_common.h"),
    "gram_gemm_kernel": ("gram.hip", "mfma_kloop.h", "device_common.h"),
}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter record, or None when the
    kernel's sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)["kernels"][kernel]
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("src_sha256_16") != source_digest(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def gram_loss_flops(N, K, n_grid):
    """MFMA flops of one Gram-form loss launch: per grid point and 256-row tile of E, column
    tile lt runs min(8 (lt + 1), K / 32) K steps of a 256 x 256 x 32 product (the lower
    triangle plus the diagonal blocks in full): ~ n_grid N K (K + 256)."""
    t = -(-K // 256)
    tiles_n = -(-N // 256)
    steps = sum(min(8 * (lt + 1), K // 32) for lt in range(t))
    return 2.0 * 256 * 256 * 32 * steps * tiles_n * n_grid


def gram_gemm_flops(M, K):
    """MFMA flops of X^T X: the t (t + 1) / 2 upper-triangle 256 x 256 tiles over the padded
    token count: ~ M K (K + 256)."""
    t = -(-K // 256)
    Mp = -(-M // 128) * 128
    return 2.0 * 256 * 256 * Mp * (t * (t + 1) // 2)


def traffic_pass():
    """Counter workload: a plain device copy of known size, then one pass of the path on a
    layer of the benchmarked shape (values drawn on the device; traffic does not depend on
    them)."""
    import torch
    import post_weight_quantization_channel_amd as awq
    dev = torch.device("cuda:0")
    src = torch.ones(1 << 29, dtype=torch.float16, device=dev)      # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log("copy of", src.numel() * 2, "bytes done")
    del src, dst
    g = torch.Generator(device=dev).manual_seed(0)
    W = (0.02 * torch.randn(N_, K_, device=dev, generator=g)).half()
    X = (torch.randn(M_, K_, device=dev, generator=g) *
         torch.exp(torch.randn(K_, device=dev, generator=g))).half()
    sx, flags = awq.act_stats(X)          # the statistics pass on its own
    for form in ("direct", "gram"):
        cfg = awq.AwqConfig(n_grid=N_GRID, form=form)
        if form == "gram":                  # as in the step: s_X from the transpose pass
            _, res = awq.stats_search_layer(W, X, cfg, flags=flags)
        else:
            res = awq.search_layer(W, X, sx, cfg, flags=flags)
        torch.cuda.synchronize()
        log(form, "search done; alpha*", int(res.best.item()))
    cr = awq.clip_search(W, X, res.s_best, cfg, flags=flags)
    p = awq.pack_int4(W, res.s_best, cfg, flags=flags, clip=cr.clip)
    awq.w4a16_gemm(torch.ones(1, K_, dtype=torch.float16, device=dev), p.qweight, p.scales16,
                   p.s16)
    torch.cuda.synchronize()
    log("path pass done")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
def w4a16_time(awq, torch, n, k, ms, group=128, zero_point=False):
    """Time W4A16 at the batch sizes `ms` on an [n, k] weight over rotated copies with HIP events.
    `us` is the GPU time per call: one pass over every copy is captured in a HIP graph and
    replayed (the result of a replay is checked against the eager calls), so the host's launch
    rate does not enter; `us_eager` is the same pass issued call by call from Python."""
    import numpy as np
    import workloads
    st = torch.cuda.current_stream()
    out = []

    def elapsed_us(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    qw, sc, s = workloads.w4a16_random_artifacts(n, k, group=group, config=4)
    zs = workloads.w4a16_random_zeros(n, k, group=group, config=4) if zero_point else None
    wbytes = qw.nbytes + sc.nbytes + (zs.nbytes if zs is not None else 0)
    copies = max(4, int(600e6 // wbytes) + 1)           # > 2 x the 256 MB Infinity Cache
    qws = [torch.from_numpy(qw.view(np.int32)).cuda() for _ in range(copies)]
    scs = [torch.from_numpy(sc).cuda() for _ in range(copies)]
    zds = [torch.from_numpy(zs).cuda() for _ in range(copies)] if zs is not None else None
    s_d = torch.from_numpy(s).cuda()
    for m in ms:
        A = torch.from_numpy(workloads.w4a16_activations(m, k, config=4)).cuda()
        Y = torch.empty((m, n), dtype=torch.float16, device="cuda")

        def one_pass():
            for i in range(copies):
                awq.w4a16_gemm(A, qws[i], scs[i], s_d, group=group, out=Y,
                               zeros=zds[i] if zds is not None else None)
        one_pass()                                      # warm-up
        torch.cuda.synchronize()
        y_eager = Y.clone()
        us_eager = elapsed_us(one_pass, 2) / copies
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            one_pass()
            side.synchronize()
            with torch.cuda.graph(graph, stream=side):
                one_pass()
        torch.cuda.synchronize()
        Y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(Y, y_eager):
            raise RuntimeError(f"W4A16 graph replay differs from the eager result (M={m})")
        us = elapsed_us(graph.replay, 3) / copies
        nbytes = (n * k // 2 + n * (k // group) * 2 + (n * (k // group) if zero_point else 0) +
                  k * 2 + m * k * 2 + m * n * 2)
        flops = 2.0 * m * n * k
        rec = {"n": n, "k": k, "m": m, "us": round(us, 3), "us_eager": round(us_eager, 3),
               "bytes": nbytes, "gbs": round(nbytes / us / 1e3, 1),
               "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
               "tflops": round(flops / us / 1e6, 2)}
        if group != 128 or zero_point:
            rec.update({"group": group, "zero_point": zero_point})
        if m >= 512:
            rec["mfma_frac"] = round(flops / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)
        out.append(rec)
        log("w4a16", rec)
        del graph
    del qws, scs, zds
    torch.cuda.empty_cache()
    return out


def w4a16_sweep(awq, torch):
    """The symmetric group-128 kernel at the batch sizes 1, 4, 16, 64, 512 for 4096x4096 and
    11008x4096."""
    out = []
    for (n, k) in ((4096, 4096), (11008, 4096)):
        out += w4a16_time(awq, torch, n, k, (1, 4, 16, 64, 512))
    return out


# ---------------------------------------------------------------------------------------------
def cpu_baseline(L, n_grid):
    """The oracle as it stands, on a bounded sample of the same layer, scaled to ms per layer.

    Sample: the activation statistics and the Gram matrix H = X^T X over the first 4096 of the
    65536 tokens (both scale linearly in the token count: x16), the quantization and the
    Gram-form loss of 2 of the 20 grid points (x10), then the argmin, the packing and one
    decode-sized W4A16 (x1)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    Ms = 4096
    Xs = L.X[:Ms]
    t = {}
    t0 = time.perf_counter()
    sx = oracle.act_stats(Xs)
    t["stats"] = (time.perf_counter() - t0) * (L.X.shape[0] / Ms)
    t0 = time.perf_counter()
    H = oracle.gram(Xs)
    t["gram"] = (time.perf_counter() - t0) * (L.X.shape[0] / Ms)
    S = oracle.scale_table(sx, n_grid)
    t0 = time.perf_counter()
    losses = []
    for i in (5, 6):
        q, d = oracle.quantize(L.W, S[i])
        losses.append(oracle.loss_gram(H, oracle.error_matrix(L.W, q, d, S[i]), Ms))
    t["alpha_points"] = (time.perf_counter() - t0) * (n_grid / 2)
    t0 = time.perf_counter()
    best = oracle.argmin_lowest(losses)
    p = oracle.pack_layer(L.W, S[5 + best])
    A = np.ones((1, L.W.shape[1]), np.float16)
    oracle.w4a16(A, p["qweight"], p["scales16"], p["s16"])
    t["pack_w4a16"] = time.perf_counter() - t0
    total_ms = 1e3 * sum(t.values())
    return {"value": round(total_ms, 1), "unit": "ms/layer", "cores": int(cores),
            "kind": "oracle",
            "sample": "stats and H=X^T X over 4096 of 65536 tokens (x16), quantize+Gram loss "
                      "for 2 of 20 alpha points (x10), argmin+pack+W4A16(M=1) once",
            "parts_ms": {k: round(1e3 * v, 1) for k, v in t.items()}}


# ---------------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.mode == "traffic":
        traffic_pass()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the "
              "path runs on one GPU (the search would shard by layer, or by output rows with one "
              "small exchange of per-grid-point loss sums)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads
    import post_weight_quantization_channel_amd as awq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    log("generating the synthetic layer (W 4096x4096 fp16, X 65536x4096 fp16) ...")
    L = workloads.c2_like_layer()
    W = torch.from_numpy(L.W).to(dev)
    X = torch.from_numpy(L.X).to(dev)
    A1 = torch.from_numpy(workloads.w4a16_activations(1, K_, config=2)).to(dev)
    cfg = awq.AwqConfig(bits=4, group=128, n_grid=N_GRID, form=args.form)
    ws_stats = torch.empty(awq.act_stats_workspace_bytes(M_, K_), dtype=torch.uint8, device=dev)
    ws_search = torch.empty(awq.search_workspace_bytes(M_, N_, K_, torch.float16, cfg),
                            dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream()

    def step(prof):
        # prof: a dict for the per-kernel durations of the search (that call then blocks until
        # the search is done), or None (nothing blocks: the timed steps). s_X and the search are
        # one call: in the Gram form the column sums come out of the pass that transposes X.
        e0, e2, e3 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(st)
        sx, res = awq.stats_search_layer(W, X, cfg, flags=flags, workspace=ws_search,
                                         stage_ms=prof)
        e2.record(st)
        p = awq.pack_int4(W, res.s_best, cfg, flags=flags)
        e3.record(st)
        Y = awq.w4a16_gemm(A1, p.qweight, p.scales16, p.s16)
        return res, (e0, e2, e3), Y

    log(f"warmup {args.warmup} step(s) ...")
    for _ in range(args.warmup):
        step({})
    torch.cuda.synchronize()

    stage_runs, ev_runs = [], []
    log(f"timing {args.steps} step(s) ...")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(st)
    for _ in range(args.steps):
        res, evs, _ = step(None)
        ev_runs.append(evs)
    t_end.record(st)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # the per-kernel breakdown of the search, from further steps outside the timed region
    for _ in range(max(3, min(args.steps, 10))):
        prof = {}
        step(prof)
        stage_runs.append(prof)
    torch.cuda.synchronize()

    # the statistics pass on its own (awq_act_stats), as context: the step takes s_X in the
    # search call instead
    stats_runs = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        awq.act_stats(X, workspace=ws_stats)
        b.record(st)
        stats_runs.append((a, b))
    torch.cuda.synchronize()
    stats_ms = statistics.mean(a.elapsed_time(b) for a, b in stats_runs[1:])
    pack_ms = statistics.mean(c.elapsed_time(d) for _, c, d in ev_runs)
    stages = {k: statistics.mean(r[k] for r in stage_runs) for k in stage_runs[0]}
    flag_bits = int(flags.item())
    losses = res.losses.cpu().numpy()
    best = int(res.best.item())
    ls = np.sort(losses)
    log(f"ms/step {ms_per_step:.3f}; stages {stages}; stats {stats_ms:.4f} ms; pack "
        f"{pack_ms:.4f} ms; alpha* {best}; flags {flag_bits}")

    def mfma_rec(kernel, ms, flops):
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(kernel), "flops_per_launch": flops,
                "launch_ms": round(ms, 4)}

    if args.form == "gram":
        mfma = [mfma_rec("gram_loss_kernel", stages["loss"], gram_loss_flops(N_, K_, N_GRID)),
                mfma_rec("gram_gemm_kernel", stages["gram_gemm"], gram_gemm_flops(M_, K_))]
    else:
        mfma = [mfma_rec("lossgemm_kernel", stages["loss"], 2.0 * M_ * N_ * K_ * N_GRID)]
    roofline = max(mfma, key=lambda r: r["launch_ms"])

    t_ = -(-K_ // 256)
    other = {
        "act_stats_standalone": {"ms": round(stats_ms, 4), "bytes": M_ * K_ * 2},
        "quantize_stack": {"ms": round(stages["quantize_stack"], 4),
                           "bytes": N_ * K_ * 2 + N_GRID * N_ * K_ * 2},
        "pack": {"ms": round(pack_ms, 4), "bytes": N_ * K_ * 2 + N_ * K_ // 2 + N_ * K_ // 64},
    }
    if args.form == "gram":
        # X read once, X^T written, plus the statistics' chunk partials
        other["x_transpose_and_stats"] = {
            "ms": round(stages["x_prep"], 4),
            "bytes": 2 * M_ * K_ * 2 + (-(-M_ // 256)) * K_ * 8}
    else:
        other["act_stats_in_search"] = {"ms": round(stages["x_prep"], 4), "bytes": M_ * K_ * 2}
    for v in other.values():
        v["gbs"] = round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)
        v["hbm_frac"] = round(v["gbs"] / HBM_PEAK_GBS, 4)

    # clipping search at s* (a further optimisation of the method, reported beside the step)
    clip_rec = None
    if args.clip_reps > 0:
        ccfg = awq.AwqConfig(bits=4, group=128, n_clip=11, clip_min=0.5)
        ws_c = torch.empty(awq.clip_workspace_bytes(M_, N_, K_, torch.float16, ccfg),
                           dtype=torch.uint8, device=dev)
        s_star = res.s_best.clone()
        times, ptimes = [], []
        for r in range(args.clip_reps + 1):            # the first run is a warm-up
            c0, c1, c2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            c0.record(st)
            cr = awq.clip_search(W, X, s_star, ccfg, workspace=ws_c)
            c1.record(st)
            awq.pack_int4(W, s_star, ccfg, clip=cr.clip)
            c2.record(st)
            c2.synchronize()
            if r:
                times.append(c0.elapsed_time(c1))
                ptimes.append(c1.elapsed_time(c2))
        ratios = cr.clip.cpu().numpy()
        clip_rec = {"n_clip": 11, "clip_min": 0.5, "ms": round(statistics.mean(times), 4),
                    "pack_clipped_ms": round(statistics.mean(ptimes), 4),
                    "groups_clipped_frac": round(float((ratios < 1.0).mean()), 4),
                    "mean_ratio": round(float(ratios.mean()), 4)}
        if args.form == "gram":
            # the same search on the operand the step's search left in its workspace
            gcfg = awq.AwqConfig(bits=4, group=128, n_grid=N_GRID, form="gram", n_clip=11,
                                 clip_min=0.5)
            gtimes = []
            for r in range(args.clip_reps + 1):
                c0, c1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                c0.record(st)
                crg = awq.clip_search_gram(W, s_star, ws_search, gcfg, flags=flags)
                c1.record(st)
                c1.synchronize()
                if r:
                    gtimes.append(c0.elapsed_time(c1))
            rg = crg.clip.cpu().numpy()
            clip_rec["after_gram_search_ms"] = round(statistics.mean(gtimes), 4)
            clip_rec["after_gram_search_same_ratio_frac"] = round(float((rg == ratios).mean()), 5)
        log("clip search", clip_rec)
        del ws_c

    # one s for three weights that read the same X (q/k/v of the attention block), and the fold
    # of s^-1 into the norm weight that produces X
    shared_rec = None
    if args.shared_reps > 0:
        del ws_search
        torch.cuda.empty_cache()
        Wk = torch.from_numpy(workloads.weight(2, N_, K_, j=1)).to(dev)
        Wv = torch.from_numpy(workloads.weight(2, N_, K_, j=2)).to(dev)
        scfg = awq.AwqConfig(bits=4, group=128, n_grid=N_GRID, form=args.form)
        ws_search = torch.empty(awq.search_workspace_bytes(M_, 3 * N_, K_, torch.float16, scfg),
                                dtype=torch.uint8, device=dev)
        gamma = torch.ones((1, K_), dtype=torch.float16, device=dev)
        t_sh, t_fold = [], []
        for r in range(args.shared_reps + 1):          # the first run is a warm-up
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record(st)
            # s_X in the same call, as in the step (awq_stats_search_layers)
            _, rs = awq.search_layers([W, Wk, Wv], X, None, scfg, workspace=ws_search)
            e1.record(st)
            awq.fold_scale(gamma, rs.s_best, axis=1)
            e2.record(st)
            e2.synchronize()
            if r:
                t_sh.append(e0.elapsed_time(e1))
                t_fold.append(e1.elapsed_time(e2))
        shared_rec = {"weights": "q, k, v: 3 x 4096x4096 fp16 sharing X", "form": args.form,
                      "search_ms": round(statistics.mean(t_sh), 3),
                      "fold_ms": round(statistics.mean(t_fold), 4),
                      "three_separate_searches_ms": round(3 * sum(stages.values()), 3),
                      "alpha_star": int(rs.best.item())}
        log("shared q/k/v search", shared_rec)
        del Wk, Wv, rs

    # zero-point codes and groups of 64: the search, the pack and W4A16 in those forms
    variants_rec = None
    if args.variant_reps > 0:
        variants_rec = []
        for (grp, zp) in ((64, False), (128, True), (64, True)):
            vcfg = awq.AwqConfig(bits=4, group=grp, n_grid=N_GRID, form=args.form,
                                 zero_point=zp)
            sx_v, _ = awq.act_stats(X, workspace=ws_stats)
            runs, tpack = [], []
            for r in range(args.variant_reps + 1):      # the first run is a warm-up
                prof = {}
                rv = awq.search_layer(W, X, sx_v, vcfg, workspace=ws_search, stage_ms=prof)
                p0, p1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
                p0.record(st)
                awq.pack_int4(W, rv.s_best, vcfg)
                p1.record(st)
                p1.synchronize()
                if r:
                    runs.append(prof)
                    tpack.append(p0.elapsed_time(p1))
            vst = {k: statistics.mean(rr[k] for rr in runs) for k in runs[0]}
            rec = {"group": grp, "zero_point": zp, "form": args.form,
                   "search_ms": round(sum(vst.values()), 3),
                   "quantize_stack_ms": round(vst["quantize_stack"], 4),
                   "loss_ms": round(vst["loss"], 4),
                   "pack_ms": round(statistics.mean(tpack), 4),
                   "alpha_star": int(rv.best.item())}
            log("variant", rec)
            rec["w4a16"] = [] if args.no_w4a16_sweep else \
                w4a16_time(awq, torch, N_, K_, (1, 512), group=grp, zero_point=zp)
            variants_rec.append(rec)

    other_form = None
    if args.other_form_reps > 0:
        oform = "direct" if args.form == "gram" else "gram"
        ocfg = awq.AwqConfig(bits=4, group=128, n_grid=N_GRID, form=oform)
        del ws_search
        torch.cuda.empty_cache()
        ws_o = torch.empty(awq.search_workspace_bytes(M_, N_, K_, torch.float16, ocfg),
                           dtype=torch.uint8, device=dev)
        sx_o, _ = awq.act_stats(X, workspace=ws_stats)
        runs = []
        for r in range(args.other_form_reps + 1):       # the first run is a warm-up
            prof = {}
            ro = awq.search_layer(W, X, sx_o, ocfg, workspace=ws_o, stage_ms=prof)
            if r:
                runs.append(prof)
        ost = {k: statistics.mean(p[k] for p in runs) for k in runs[0]}
        lo = ro.losses.cpu().numpy()
        if oform == "direct":
            orec = mfma_rec("lossgemm_kernel", ost["loss"], 2.0 * M_ * N_ * K_ * N_GRID)
        else:
            orec = mfma_rec("gram_loss_kernel", ost["loss"], gram_loss_flops(N_, K_, N_GRID))
        other_form = {"form": oform, "search_ms": round(sum(ost.values()), 3),
                      "alpha_star": int(ro.best.item()),
                      "max_loss_rel_diff": float(np.max(np.abs(lo - losses) / losses)),
                      "loss_kernel": orec, "stages_ms": {k: round(v, 4) for k, v in ost.items()}}
        log("other form", other_form)
        del ws_o
    else:
        del ws_search

    del X
    torch.cuda.empty_cache()
    w4 = [] if args.no_w4a16_sweep else w4a16_sweep(awq, torch)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample) ...")
        cpu = cpu_baseline(L, N_GRID)
        log("cpu baseline", cpu)

    line = {
        "metric": "AWQ search ms per 4096x4096 layer + % MFMA peak; W4A16 GEMV HBM GB/s",
        "value": round(ms_per_step, 3), "unit": "ms/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama7b_attn_proj_4096x4096_tokens65536_int4_g128_grid20",
                   "N": N_, "K": K_, "M": M_, "bits": 4, "group": 128, "n_grid": N_GRID,
                   "w4a16_decode_m": 1, "search_form": args.form},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "search_form": args.form,
        "mfma": mfma,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "other_form": other_form,
        "clip_search": clip_rec,
        "shared_qkv": shared_rec,
        "quant_variants": variants_rec,
        "hbm_stages": other,
        "w4a16": w4,
        "alpha_star": best,
        "loss_gap": float((ls[1] - ls[0]) / ls[0]),
        "flags": flag_bits,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
