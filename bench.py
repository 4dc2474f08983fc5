#!/usr/bin/env python3
"""Benchmark of the AWQ hot path on one MI355X.

One step = one pass of the whole path over the LLaMA-7B-shaped attention projection (W fp16
4096x4096, 65536 calibration tokens = 128 samples x 512 tokens, INT4, group 128, 20 alpha points):
    awq_stats_search_layer (s_X, then the alpha search) -> awq_pack_int4(s*) -> w4a16_gemm
    (decode, M = 1).
The search runs in the Gram form (H = X^T X once, read straight from fp16 X, then one K x K
contraction per grid point), and s_X comes from the statistics pass inside the same call
(awq_act_stats alone is timed as context);
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
  w4a16         w4a16_gemm_ws at the batch sizes 1, 4, 16, 64, 128, 512 for 4096x4096 and
                11008x4096 (and 1, 16 for 8192x8192, 28672x8192, 8192x28672), over rotated
                weight copies (> 256 MB, so HBM and not the
                Infinity Cache is measured), replayed from a HIP graph (GPU time per call;
                `us_eager`: the same calls issued one by one from Python): GB/s and fraction
                of 8 TB/s (TFLOP/s and MFMA fraction at M = 512);
  cpu_baseline  the CPU oracle on a bounded sample of the same layer, scaled to ms per layer;
  layers        the other layer shapes of the workloads, each searched (s_X in the same call,
                Gram form, 20 alpha points) and packed like the step: the LLaMA-7B MLP trio
                (gate and up 11008x4096 sharing one X, down 4096x11008 with its own X) and the
                70B-class shapes (8192x8192, 1024x8192, 28672x8192 on one X of 8192 channels)
                in INT4 and INT3: ms per layer, the kernel breakdown, the MFMA fractions of the
                two contractions (on executed and on strict-triangle flops), and the oracle's
                time for the layer scaled from the step's CPU sample (not run: minutes each);
                plus gate and up searched together (one s) and an estimate for one LLaMA-7B
                decoder block and a 32-block model, as context.
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
    ap.add_argument("--layer-reps", type=int, default=2,
                    help="repetitions of each other layer shape's search (0: skip them)")
    ap.add_argument("--counters", default=None,
                    help="record mode: directory holding one rocprofv3 CSV directory per pass")
    ap.add_argument("--mode", choices=("bench", "traffic", "record", "ceilings"), default="bench",
                    help="traffic: one 1 GiB device copy (counter calibration) and one pass of "
                         "the path in each form, for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs")
    return ap.parse_args()


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "search_c2_traffic.json")
CSRC = os.path.join(ROOT, "post_weight_quantization_channel_amd", "csrc")
# the sources each MFMA kernel is compiled from (a counter record is valid only for these bytes)
KERNEL_SOURCES = {
    "lossgemm_kernel": ("lossgemm.hip", "mfma_kloop.h", "device_common.h"),
    "gram_loss_kernel": ("gram.hip", "mfma_kloop.h", "device_common.h"),
    "gram_gemm_x_kernel": ("gram.hip", "mfma_kloop.h", "device_common.h"),
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
    """The method's flops in one Gram-form loss launch: the quadratic form E H E^T of every grid
    point with H symmetric, one multiply-add per pair of channels and weight row, i.e.
    n_grid N K^2 (the strict triangle; the diagonal adds n_grid N K more)."""
    return float(n_grid) * N * K * K


def gram_loss_executed_flops(N, K, n_grid):
    """MFMA flops the Gram-form loss kernel issues: per grid point and 256-row tile of E, column
    tile lt runs nk = min(8 (lt + 1), K / 32) K steps of a 256 x 256 x 32 product. In a full tile
    the last eight steps cover the diagonal block of the lower-triangular operand, and step d
    of them (d = 0..7) issues only the products of its 8 - d live 32-column blocks (36 of 64 in
    all, i.e. 4.5 steps' worth); the ragged last tile runs all its steps in full."""
    t = -(-K // 256)
    tiles_n = -(-N // 256)
    steps = 0.0
    for lt in range(t):
        nk = min(8 * (lt + 1), K // 32)
        steps += (nk - 8 + 4.5) if nk == 8 * (lt + 1) else nk
    return 2.0 * 256 * 256 * 32 * steps * tiles_n * n_grid


def gram_gemm_flops(M, K):
    """The method's flops of H = X^T X: one multiply-add per token and pair of channels of the
    symmetric product, M K^2."""
    return float(M) * K * K


def gram_gemm_executed_flops(M, K):
    """MFMA flops of X^T X as the kernel runs it: the t (t + 1) / 2 upper-triangle 256 x 256
    tiles over the padded token count: ~ M K (K + 256)."""
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
        if form == "gram":                  # as in the step: s_X inside the search call
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
    # W4A16 on random artefacts of the two LLaMA-7B shapes, one call per batch size, in this
    # order (the counter record matches dispatches to these calls by order)
    for n, k, m, ws in W4A16_COUNTER_CALLS:
        qw = torch.randint(-2**31, 2**31 - 1, (n, k // 8), dtype=torch.int32, device=dev,
                           generator=g)
        sc = (0.01 * torch.rand(n, k // 128, device=dev, generator=g) + 1e-3).half()
        s16 = (1.0 + torch.rand(k, device=dev, generator=g)).half()
        A = torch.randn(m, k, device=dev, generator=g).half()
        if ws:
            wsp = torch.empty(max(1, awq.w4a16_gemm_workspace_bytes(m, n, k)), dtype=torch.uint8,
                              device=dev)
            awq.w4a16_gemm_ws(A, qw, sc, s16, workspace=wsp)
        else:
            awq.w4a16_gemm(A, qw, sc, s16)
        torch.cuda.synchronize()
    log("w4a16 calls done")


def ceiling_pass(sizes=(1 << 30, M_ * K_ * 2, N_GRID * N_ * K_ * 2), reps=20, echo=True):
    """Reference rates of plain streams on this GPU, with torch's own elementwise and reduction
    kernels over fp16 buffers, HIP events on the current stream: a write-only fill, a copy, and a
    read-only reduction, by default at 1 GiB and at the sizes of the path's bandwidth-bound
    kernels (the 65536 x 4096 fp16 activations, 537 MB; the 20 x 4096 x 4096 fp16 error stack,
    671 MB)."""
    import torch
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    out = []
    for nbytes in sizes:
        src = torch.ones(nbytes // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        acc = torch.empty((), dtype=torch.float32, device=dev)
        ops = {"write (fill_)": (lambda: dst.fill_(2.0), nbytes),
               "copy (copy_)": (lambda: dst.copy_(src), 2 * nbytes),
               "read (sum to fp32)": (lambda: torch.sum(src, dim=0, dtype=torch.float32, out=acc),
                                         nbytes)}
        for name, (fn, moved) in ops.items():
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                fn()
            e1.record(st)
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            rec = {"op": name, "bytes": nbytes, "moved": moved, "us": round(us, 1),
                   "gbs": round(moved / us / 1e3, 1),
                   "hbm_frac": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)}
            if echo:
                print(json.dumps(rec), flush=True)
            out.append(rec)
        del src, dst
        torch.cuda.empty_cache()
    return out


# (n, k, m, through w4a16_gemm_ws) of the W4A16 calls of the counter pass; a call on K slices
# is two dispatches (the slices, then their sum)
W4A16_COUNTER_CALLS = [(4096, 4096, 1, False), (4096, 4096, 16, False), (4096, 4096, 64, False),
                       (4096, 4096, 64, True), (4096, 4096, 128, True), (4096, 4096, 512, False),
                       (11008, 4096, 1, False), (11008, 4096, 4, False), (11008, 4096, 16, False),
                       (11008, 4096, 64, True), (28672, 8192, 1, False)]
W4A16_SUM_KERNELS = ("w4a16_splitk_reduce_kernel", "w4a16_sum_slices_kernel")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "awq_path_c2_counters.txt")
COUNTER_PASSES = {
    "trace": "--kernel-trace --stats",
    "fetch": "--pmc FETCH_SIZE",
    "write": "--pmc WRITE_SIZE",
    "mfma": "--pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES "
            "SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE",
}


def record_counters(ctr_dir):
    """Write the counter record that `measured_traffic` reads and its text summary from the CSV
    output of rocprofv3 passes over `bench.py --mode traffic`: one directory per pass under
    `ctr_dir` (trace, fetch, write, mfma), each made by
        rocprofv3 <pass counters> --output-format csv -d <ctr_dir>/<pass> -o t \
            -- python3 bench.py --mode traffic
    Every pass runs the same launches in the same order, so dispatch ids match across passes
    (checked by kernel name). Byte counters are scaled by what they read for the 1 GiB copy."""
    import csv
    import collections

    def load(sub, fname):
        with open(os.path.join(ctr_dir, sub, fname)) as f:
            return list(csv.DictReader(f))

    def counters(sub):
        vals, names, grid = collections.defaultdict(dict), {}, {}
        for r in load(sub, "t_counter_collection.csv"):
            i = int(r["Dispatch_Id"])
            names[i], grid[i] = r["Kernel_Name"], int(r["Grid_Size"])
            vals[i][r["Counter_Name"]] = vals[i].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return vals, names, grid

    dur, tnames = {}, {}
    for r in load("trace", "t_kernel_trace.csv"):
        i = int(r["Dispatch_Id"])
        dur[i] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        tnames[i] = r["Kernel_Name"]
    fetch, fnames, grid = counters("fetch")
    write, wnames, _ = counters("write")
    mfma, mnames, _ = counters("mfma")
    for i, n in tnames.items():
        for other in (fnames, wnames, mnames):
            if i in other and other[i] != n:
                raise RuntimeError(f"dispatch {i}: {n} vs {other[i]} (passes out of step)")
    copies = [i for i, n in fnames.items() if "copyBuffer" in n]
    big = max(copies, key=lambda i: fetch[i]["FETCH_SIZE"])
    rf = (1 << 30) / (fetch[big]["FETCH_SIZE"] * 1024.0)
    wf = (1 << 30) / (write[big]["WRITE_SIZE"] * 1024.0)

    def short(name):
        name = name.replace("void ", "").replace("awq::", "")
        cut = name.find("(")
        return name[:cut] if cut > 0 else name

    t_ = -(-K_ // 256)
    algo = {"lossgemm_kernel": M_ * K_ * 2 + N_GRID * N_ * K_ * 2,
            "gram_loss_kernel": N_GRID * N_ * K_ * 2 + K_ * K_ * 2}
    w4_calls = iter(W4A16_COUNTER_CALLS)
    rows, kernels = [], {}
    seen_w4 = 0
    call_label = ""
    for i in sorted(tnames):
        n = short(tnames[i])
        if "awq" not in tnames[i] and i != big:
            continue
        if i not in fetch or i not in write or i not in mfma:
            continue
        fb = fetch[i]["FETCH_SIZE"] * 1024.0 * rf
        wb = write[i]["WRITE_SIZE"] * 1024.0 * wf
        c = mfma[i]
        cyc = c["GRBM_GUI_ACTIVE"] / 8.0           # the counter sums the 8 XCDs
        us = dur[i]
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / cyc if cyc else 0.0   # 1024 SIMDs
        label = n
        a_bytes = algo.get(n)
        if n == "gram_gemm_x_kernel":
            # X read once plus the fp32 partial tiles written, one 256 x 256 tile per workgroup
            a_bytes = M_ * K_ * 2 + (grid[i] // 256) * 256 * 256 * 4
        if n.startswith(W4A16_SUM_KERNELS):
            label = f"{call_label}: {n}"           # the second dispatch of a call on K slices
        elif n.startswith("w4a16") and seen_w4 >= 1:
            nn, kk, mm, ws = next(w4_calls)
            call_label = f"w4a16{'_ws' if ws else ''} {nn}x{kk} M={mm}"
            label = f"{call_label}: {n}"
            a_bytes = nn * kk // 2 + nn * (kk // 128) * 2 + kk * 2 + mm * kk * 2 + mm * nn * 2
        if n.startswith("w4a16"):
            seen_w4 += 1                           # the first is the path pass's decode call
        rows.append((i, label, grid[i], us, fb, wb, a_bytes, c["SQ_INSTS_MFMA"], busy,
                     cyc / us / 1e3 if us > 0 else 0.0))
        if n in ("lossgemm_kernel", "gram_loss_kernel", "gram_gemm_x_kernel") and n not in kernels:
            kernels[n] = {"fetch_kib": fetch[i]["FETCH_SIZE"], "write_kib": write[i]["WRITE_SIZE"],
                          "hbm_bytes_per_launch": int(fb + wb),
                          "algorithmic_bytes_per_launch": int(a_bytes),
                          "mfma_insts": int(c["SQ_INSTS_MFMA"]), "mfma_busy": round(busy, 4),
                          "clock_ghz": round(cyc / us / 1e3, 3), "trace_us": round(us, 1),
                          "src_sha256_16": source_digest(n)}
    cmds = [f"rocprofv3 {v} --output-format csv -d <dir>/{k} -o t -- python3 bench.py --mode traffic"
            for k, v in COUNTER_PASSES.items()]
    rec = {"workload": f"{N_}x{K_} fp16 layer, {M_} fp16 tokens, {N_GRID} alpha points; "
                       "W4A16 calls " + ", ".join(f"{'w4a16_gemm_ws' if w else 'w4a16_gemm'} {n}x{k} M={m}"
                                      for n, k, m, w in W4A16_COUNTER_CALLS),
           "read_factor": rf, "write_factor": wf, "commands": cmds, "kernels": kernels}
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
    lines = [
        "# rocprofv3 counters of one pass of the path (bench.py --mode traffic): a 1 GiB device",
        f"# copy, the search of a {N_}x{K_} fp16 layer with {M_} fp16 tokens at {N_GRID} grid points",
        "# in each form (direct, Gram), clipping search, pack, one decode call, then W4A16 calls on",
        "# random artefacts (shapes in brackets).",
        "#",
        "# commands (from /tmp, TMPDIR=/tmp), one run per pass:",
    ] + [f"#   {c}" for c in cmds] + [
        "# then: python3 bench.py --mode record --counters <dir>",
        "#",
        f"# read factor {rf:.4f}, write factor {wf:.4f} (FETCH_SIZE / WRITE_SIZE of the 1 GiB copy);",
        "# the byte counters count traffic leaving L2 toward memory (Infinity Cache hits included).",
        "# us: kernel-trace duration of the same dispatch (trace pass). clock: GRBM_GUI_ACTIVE / 8",
        "# XCDs / us (meaningless for dispatches of a few us, where the counter window dominates).",
        "# mfma_busy: SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8); busy x clock is",
        "# the MFMA rate in units of one SIMD fully busy at 1 GHz (2.4 = the 2.5 PFLOP/s peak).",
        "",
        f"{'dispatch':>8} {'kernel':66s} {'grid':>10} {'us':>10} {'read_MB':>10} {'write_MB':>9} "
        f"{'algo_MB':>9} {'ratio':>6} {'mfma_insts':>11} {'busy':>6} {'clock':>6} {'busyxclk':>8}",
    ]
    for (i, label, g, us, fb, wb, ab, mi, busy, clk) in rows:
        ratio = f"{(fb + wb) / ab:6.2f}" if ab else "     -"
        amb = f"{ab / 1e6:9.1f}" if ab else "        -"
        lines.append(f"{i:8d} {label[:66]:66s} {g:10d} {us:10.1f} {fb / 1e6:10.1f} {wb / 1e6:9.1f} "
                     f"{amb} {ratio} {int(mi):11d} {busy:6.3f} {clk:6.2f} {busy * clk:8.3f}")
    with open(COUNTER_SUMMARY, "w") as f:
        f.write("\n".join(lines) + "\n")
    log("wrote", TRAFFIC_RECORD, "and", COUNTER_SUMMARY)


# ---------------------------------------------------------------------------------------------
def w4a16_time(awq, torch, n, k, ms, group=128, zero_point=False, ws=True, with_s=True):
    """Time W4A16 at the batch sizes `ms` on an [n, k] weight over rotated copies with HIP events.
    `us` is the GPU time per call: one pass over every copy is captured in a HIP graph and
    replayed (the result of a replay is checked against the eager calls), so the host's launch
    rate does not enter; `us_eager` is the same pass issued call by call from Python.
    ws: w4a16_gemm_ws with one workspace (K split over workgroups where it pays), else
    w4a16_gemm. with_s False: s16 = NULL (s folded into the producer of A)."""
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
    s_d = torch.from_numpy(s).cuda() if with_s else None
    for m in ms:
        A = torch.from_numpy(workloads.w4a16_activations(m, k, config=4)).cuda()
        Y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        wsp = torch.zeros(max(1, awq.w4a16_gemm_workspace_bytes(m, n, k, group)),
                          dtype=torch.uint8, device="cuda")

        def one_pass():
            for i in range(copies):
                if ws:
                    awq.w4a16_gemm_ws(A, qws[i], scs[i], s_d, group=group, out=Y,
                                      zeros=zds[i] if zds is not None else None, workspace=wsp)
                else:
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
                  (k * 2 if with_s else 0) + m * k * 2 + m * n * 2)
        flops = 2.0 * m * n * k
        rec = {"n": n, "k": k, "m": m, "entry": "w4a16_gemm_ws" if ws else "w4a16_gemm",
               "us": round(us, 3), "us_eager": round(us_eager, 3),
               "bytes": nbytes, "gbs": round(nbytes / us / 1e3, 1),
               "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
               "tflops": round(flops / us / 1e6, 2)}
        if group != 128 or zero_point:
            rec.update({"group": group, "zero_point": zero_point})
        if not with_s:
            rec["s16"] = None
        if m >= 512:
            rec["mfma_frac"] = round(flops / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)
        out.append(rec)
        log("w4a16", rec)
        del graph
    del qws, scs, zds
    torch.cuda.empty_cache()
    return out


def layer_sweep(awq, torch, reps, cpu_parts):
    """The MLP trio of LLaMA-7B and the 70B-class shapes through the step's search and pack
    (s_X in the same call, Gram form): ms per layer, kernel breakdown and MFMA fractions; the
    oracle's time scaled from the C2 sample (`cpu_parts`: its parts in ms, or None)."""
    import numpy as np
    import workloads
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()

    def oracle_estimate(n, k):
        # the oracle's parts at C2 scale as: statistics M K, H = X^T X  M K^2, the 20 grid
        # points N K^2 (the loss contraction dominates), packing N K
        if not cpu_parts:
            return None
        f = k / K_
        est = (cpu_parts["stats"] * f + cpu_parts["gram"] * f * f +
               cpu_parts["alpha_points"] * (n / N_) * f * f + cpu_parts["pack_w4a16"] * (n / N_) * f)
        return {"ms_estimate": round(est, 0), "run": False,
                "why": "scaled from the step's oracle sample (each layer would take minutes of "
                       "host time; the benchmark keeps to a few minutes)"}

    def one(name, Wt, Xt, bits, n, k):
        cfg = awq.AwqConfig(bits=bits, group=128, n_grid=N_GRID, form="gram")
        ws = torch.empty(awq.search_workspace_bytes(M_, n, k, torch.float16, cfg),
                         dtype=torch.uint8, device=dev)
        times = []
        for r in range(reps + 1):                      # the first run is a warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            sx, res = awq.stats_search_layer(Wt, Xt, cfg, workspace=ws)
            awq.pack_int4(Wt, res.s_best, cfg)
            e1.record(st)
            e1.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        prof = {}
        sx, res = awq.stats_search_layer(Wt, Xt, cfg, workspace=ws, stage_ms=prof)
        losses = np.sort(res.losses.cpu().numpy())
        fl_loss = gram_loss_flops(n, k, N_GRID)
        ex_loss = gram_loss_executed_flops(n, k, N_GRID)
        fl_gemm = gram_gemm_flops(M_, k)
        ex_gemm = gram_gemm_executed_flops(M_, k)

        def frac(fl, ms):
            return round(fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
        rec = {"layer": name, "N": n, "K": k, "M": M_, "bits": bits,
               "ms": round(statistics.mean(times), 3),
               "stages_ms": {kk: round(v, 4) for kk, v in prof.items()},
               "gram_loss": {"ms": round(prof["loss"], 4),
                             "frac": frac(fl_loss, prof["loss"]),
                             "frac_executed": frac(ex_loss, prof["loss"])},
               "gram_gemm": {"ms": round(prof["gram_gemm"], 4),
                             "frac": frac(fl_gemm, prof["gram_gemm"]),
                             "frac_executed": frac(ex_gemm, prof["gram_gemm"])},
               "alpha_star": int(res.best.item()),
               "loss_gap": float((losses[1] - losses[0]) / losses[0]),
               "flags": int(res.flags.item()),
               "oracle": oracle_estimate(n, k)}
        log("layer", rec)
        del ws
        torch.cuda.empty_cache()
        return rec

    out = []
    log("generating the LLaMA-7B MLP trio (X 65536x4096 and 65536x11008 fp16) ...")
    gate, up, down = workloads.c3_layers(m=M_)
    Xg = torch.from_numpy(gate.X).to(dev)
    Wg = torch.from_numpy(gate.W).to(dev)
    Wu = torch.from_numpy(up.W).to(dev)
    out.append(one("llama7b_mlp_gate_11008x4096", Wg, Xg, 4, 11008, 4096))
    out.append(one("llama7b_mlp_up_11008x4096", Wu, Xg, 4, 11008, 4096))
    # gate and up read the same X: one s for both (awq_stats_search_layers)
    cfg = awq.AwqConfig(bits=4, group=128, n_grid=N_GRID, form="gram")
    ws = torch.empty(awq.search_workspace_bytes(M_, 2 * 11008, 4096, torch.float16, cfg),
                     dtype=torch.uint8, device=dev)
    gu = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        _, rgu = awq.search_layers([Wg, Wu], Xg, None, cfg, workspace=ws)
        awq.pack_int4(Wg, rgu.s_best, cfg)
        awq.pack_int4(Wu, rgu.s_best, cfg)
        e1.record(st)
        e1.synchronize()
        if r:
            gu.append(e0.elapsed_time(e1))
    gateup = {"layer": "llama7b_mlp_gate+up_shared_s", "ms": round(statistics.mean(gu), 3),
              "alpha_star": int(rgu.best.item())}
    log("layer", gateup)
    del ws, Xg, Wg, Wu, gate, up
    torch.cuda.empty_cache()
    Xd = torch.from_numpy(down.X).to(dev)
    Wd = torch.from_numpy(down.W).to(dev)
    out.append(one("llama7b_mlp_down_4096x11008", Wd, Xd, 4, 4096, 11008))
    del Xd, Wd, down
    torch.cuda.empty_cache()

    log("generating the 70B-class activations (X 65536x8192 fp16) ...")
    X5 = torch.from_numpy(workloads.c5_x(m=M_)).to(dev)
    for (n, j, nm) in ((8192, 0, "attn_8192x8192"), (1024, 1, "gqa_kv_1024x8192"),
                       (28672, 3, "mlp_28672x8192")):
        W5 = torch.from_numpy(workloads.c5_weight(n, j=j)).to(dev)
        for bits in (4, 3):
            out.append(one(f"70b_{nm}_int{bits}", W5, X5, bits, n, 8192))
        del W5
        torch.cuda.empty_cache()
    del X5
    torch.cuda.empty_cache()
    return out, gateup


def w4a16_sweep(awq, torch):
    """w4a16_gemm_ws, symmetric codes in groups of 128, at the batch sizes 1, 2, 4, 16, 64, 128,
    512 for 4096x4096 and 11008x4096, and at 1 and 16 for the 70B-class shapes 8192x8192,
    28672x8192 and 8192x28672 (decode GB/s where the weight is large enough to stream)."""
    out = []
    for (n, k) in ((4096, 4096), (11008, 4096)):
        out += w4a16_time(awq, torch, n, k, (1, 2, 4, 16, 64, 128, 512))
    for (n, k) in ((8192, 8192), (28672, 8192), (8192, 28672)):
        out += w4a16_time(awq, torch, n, k, (1, 16))
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
    # the host cores this process may run on; the BLAS pool is sized to them (capped by the
    # OMP_NUM_THREADS share the host gives a job, when set), and `cores` is what it used
    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover
        limiter = None
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
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": round(total_ms, 1), "unit": "ms/layer", "cores": int(cores),
            "affinity_cores": affinity,
            "kind": "oracle",
            "sample": "stats and H=X^T X over 4096 of 65536 tokens (x16), quantize+Gram loss "
                      "for 2 of 20 alpha points (x10), argmin+pack+W4A16(M=1) once",
            "parts_ms": {k: round(1e3 * v, 1) for k, v in t.items()}}


# ---------------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.mode == "record":
        record_counters(args.counters)
        return
    if args.mode == "ceilings":
        ceiling_pass()
        return
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
        # one call.
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

    def mfma_rec(kernel, ms, flops, executed=None):
        # achieved: the method's flops (n N K^2 for the loss, M K^2 for X^T X; N M K per grid
        # point for the direct form); the flops the kernel issues are reported beside them
        achieved = flops / (ms * 1e-3) / 1e12
        rec = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 1),
               "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
               "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
               "traffic": measured_traffic(kernel), "flops_per_launch": flops,
               "launch_ms": round(ms, 4)}
        if executed is not None:
            rec["executed_flops_per_launch"] = executed
            rec["frac_executed"] = round(executed / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
        return rec

    if args.form == "gram":
        mfma = [mfma_rec("gram_loss_kernel", stages["loss"], gram_loss_flops(N_, K_, N_GRID),
                         gram_loss_executed_flops(N_, K_, N_GRID)),
                mfma_rec("gram_gemm_x_kernel", stages["gram_gemm"], gram_gemm_flops(M_, K_),
                         gram_gemm_executed_flops(M_, K_))]
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
    # fp16 X: both forms read X as it is, so the search's first stage is the statistics pass
    other["act_stats_in_search"] = {"ms": round(stages["x_prep"], 4), "bytes": M_ * K_ * 2}
    for v in other.values():
        v["gbs"] = round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)
        v["hbm_frac"] = round(v["gbs"] / HBM_PEAK_GBS, 4)
    # the stream rates this GPU reaches with torch's own fill and copy kernels at these sizes:
    # read-dominated stages against the copy, the write-dominated error stack against the fill
    rates = {(r["op"].split()[0], r["bytes"]): r["gbs"]
             for r in ceiling_pass(sizes=(M_ * K_ * 2, N_GRID * N_ * K_ * 2), reps=10, echo=False)}
    ceil_of = {"act_stats_standalone": ("copy", M_ * K_ * 2),
               "act_stats_in_search": ("copy", M_ * K_ * 2),
               "quantize_stack": ("write", N_GRID * N_ * K_ * 2)}
    for k, v in other.items():
        if k in ceil_of:
            op, nb = ceil_of[k]
            v["stream_ceiling"] = {"op": "torch " + ("fill_" if op == "write" else "copy_"),
                                   "bytes": nb, "gbs": rates[(op, nb)]}
            v["vs_ceiling"] = round(v["gbs"] / rates[(op, nb)], 4)
    # quantize_stack is bound by its vector ALU work (the quantizer at 20 grid points per weight:
    # about 13 VALU instructions per element, the VALU busy for ~92% of the kernel in the counter
    # record); pack moves 42 MB in a single short launch
    other["quantize_stack"]["bound"] = "alu"
    other["pack"]["bound"] = "launch"

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
            orec = mfma_rec("gram_loss_kernel", ost["loss"], gram_loss_flops(N_, K_, N_GRID),
                            gram_loss_executed_flops(N_, K_, N_GRID))
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
    del L

    layers, block = None, None
    if args.layer_reps > 0:
        layers, gateup = layer_sweep(awq, torch, args.layer_reps,
                                     cpu["parts_ms"] if cpu else None)
        # one LLaMA-7B decoder block: q/k/v with one s, o (the step's layer), gate/up with one
        # s, down; the pages quote about 3 minutes (and about 2) for a whole 7B model, on
        # hardware they do not state
        down_ms = next(r["ms"] for r in layers if r["layer"].startswith("llama7b_mlp_down"))
        if shared_rec is not None:
            block_ms = shared_rec["search_ms"] + ms_per_step + gateup["ms"] + down_ms
            block = {"block_ms": round(block_ms, 2), "model_32_blocks_s": round(32 * block_ms / 1e3, 2),
                     "parts": {"qkv_shared": shared_rec["search_ms"], "o": round(ms_per_step, 3),
                               "gate_up_shared": gateup["ms"], "down": down_ms},
                     "note": "context only: calibration activations of each layer resident on "
                             "the GPU; excludes running the model to collect them"}

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
        "layers": layers,
        "llama7b_block_estimate": block,
        "alpha_star": best,
        "loss_gap": float((ls[1] - ls[0]) / ls[0]),
        "flags": flag_bits,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
