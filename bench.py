#!/usr/bin/env python3
"""Benchmark: sparse top-k MoE FFN layer forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config c5] [--no-cpu-baseline]

A step is one moe_forward (router + losses, dispatch, expert FFN up and down,
combine) over one batch of seeded synthetic input that is already resident in
HBM.  The default workload is the Mixtral-8x7B-shaped layer (T=16384 tokens,
H=4096, 8 experts, top-2, FFN 14336, capacity factor 2.0, bf16 storage, fp32
accumulation).  Prints ONE JSON line.

value         tokens/s = T * K / (timed wall time of K back-to-back steps)
roofline      the dominant kernel (the larger FFN GEMM) against its bound: the
              dense bf16 MFMA peak (achieved = 2*A*H*F flop per launch / its
              mean duration from HIP events the library records on its own
              stream), or HBM bandwidth when the launch's algorithmic bytes
              (weights of the experts with rows, A input and output rows) take
              longer at 8 TB/s than its flops at the MFMA peak (few tokens)
cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/s and FFN TFLOP/s (% bf16 MFMA peak) on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c5")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--train", action="store_true",
                    help="time a training step instead: moe_forward_train then moe_backward "
                         "(aux and z loss weights 0.01 and 0.001), one JSON line")
    ap.add_argument("--no-vendor-reference", action="store_true",
                    help="skip the same-machine side references appended to the JSON line "
                         "(the vendor batched GEMM on the expert shapes, plain streams over x)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the forward replayed as a captured HIP graph")
    ap.add_argument("--no-abi-timing", action="store_true",
                    help="skip the per-call warm/cold timing that follows the timed steps "
                         "(thousands of extra launches; counter runs of the profiler omit it)")
    ap.add_argument("--cpu-seconds", type=float, default=90.0,
                    help="the oracle runs the whole forward when a probe predicts at most this "
                         "many seconds, else a token prefix of about this much work")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before timing, run one plain device-to-device copy of MIB MiB "
                         "(the reference kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    ap.add_argument("--vendor-gemm", type=float, default=0.0, metavar="SECONDS",
                    help="instead of the layer: time the vendor library's batched GEMM "
                         "(torch.bmm, hipBLASLt) on the workload's two expert GEMM shapes with "
                         "balanced experts, each for about SECONDS, one JSON line (a side "
                         "reference for the expert GEMMs; the library is not called)")
    ap.add_argument("--vendor-stream", type=float, default=0.0, metavar="SECONDS",
                    help="instead of the layer: time the runtime's device-to-device copy and "
                         "torch's sum over a buffer the size of the workload's x, each for "
                         "about SECONDS, one JSON line (the practical HBM rate the router's "
                         "read of x is held against; the library is not called)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, "
                         "WRITE_SIZE, both with --calibrate-copy) into "
                         "profiles/traffic_<workload>.json")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of every kernel and host source of the library: traffic figures taken
    on other sources are not reported."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_mixture_experts_21_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current sources and the same workload."""
    try:
        with open(traffic_path(workload)) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash() or d.get("workload") != workload:
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if not k else k.get("hbm_bytes")


def kernel_key(symbol: str) -> str:
    """Short name of a kernel symbol: the expert GEMM as up / down (template
    arguments <BM, activation, save>: activation 0 is the second GEMM), else
    the function name."""
    base = symbol.replace("(anonymous namespace)::", "").split("(")[0]
    name = base.split("<")[0].split("::")[-1].strip()
    if name == "ffn_gemm_bf16":
        targs = [a.strip() for a in base.split("<", 1)[1].split(">")[0].split(",")]
        return "ffn_gemm_bf16_down" if targs[1] == "0" else "ffn_gemm_bf16_up"
    return name


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, copy_mib: int = 256):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel of the run,
    scaled by what the same counters read for the calibration copy of known
    size, in bytes per launch."""
    import csv
    import glob

    def per_kernel(d, counter):
        # mean per dispatch, keyed by kernel; the calibration copy is the copy
        # dispatch with the largest grid
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        acc, copy = {}, (0, None)
        for r in rows:
            v, g = float(r["Counter_Value"]), int(r["Grid_Size"])
            if "copyBuffer" in r["Kernel_Name"]:
                if g > copy[0]:
                    copy = (g, v)
                continue
            if "fill" in r["Kernel_Name"] or "elementwise" in r["Kernel_Name"]:
                continue
            acc.setdefault(kernel_key(r["Kernel_Name"]), []).append(v)
        return {k: sum(v) / len(v) for k, v in acc.items()}, copy[1]

    (fetch, c_fetch), (write, c_write) = (per_kernel(fetch_dir, "FETCH_SIZE"),
                                          per_kernel(write_dir, "WRITE_SIZE"))
    if c_fetch is None or c_write is None:
        raise SystemExit("no calibration copy kernel found in the pmc runs")
    kib = copy_mib * 1024.0
    f_fetch, f_write = c_fetch / kib, c_write / kib
    out = {"source_hash": kernel_source_hash(), "workload": workload,
           "calibration_kernel": "__amd_rocclr_copyBuffer", "calibration_copy_kib": kib,
           "fetch_factor": f_fetch, "write_factor": f_write, "kernels": {}}
    lines = ["| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (scaled) |",
             "|---|---|---|---|"]
    for k in sorted(fetch, key=lambda n: -fetch[n]):
        hbm = (fetch[k] / f_fetch + write.get(k, 0.0) / f_write) * 1024.0
        out["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write.get(k), "hbm_bytes": hbm}
        lines.append(f"| {k} | {fetch[k]:.0f} | {write.get(k, 0):.0f} | {hbm:.4g} |")
    return out, lines


def vendor_gemm(spec, seconds: float):
    """torch.bmm (hipBLASLt) on the expert GEMM shapes of `spec` with every
    expert holding T k / E rows: [E, M, H] x [E, H, F] and [E, M, F] x [E, F, H]
    in bf16, inputs drawn like the layer's (rows N(0, 1), weights N(0, 0.02)).
    No activation, no gather and no ragged groups, so it is a plain batched
    GEMM of the same flops: context for the expert GEMMs' rate, not the path."""
    import torch
    E, H, F = spec.E, spec.H, spec.F
    M = spec.T * spec.k // E
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    res = {"workload": spec.name, "rows_per_expert": M, "kernel": "torch.bmm (hipBLASLt)"}
    for name, (K, N) in (("up", (H, F)), ("down", (F, H))):
        a = torch.randn(E, M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(E, K, N, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
        c = torch.bmm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n, t0 = 0, time.perf_counter()
        e0.record()
        while n < 3 or time.perf_counter() - t0 < seconds:
            for _ in range(10):
                torch.bmm(a, b, out=c)
            n += 10
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        flops = 2.0 * E * M * K * N
        res[name] = {"calls": n, "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                     "frac_of_bf16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        del a, b, c
    return res


def vendor_stream(spec, seconds: float):
    """Plain streams over a buffer of the workload's x size (T x H bf16): the
    runtime's device-to-device copy (reads and writes every byte) and torch's
    sum (reads every byte once), each timed with HIP events over back-to-back
    calls."""
    import torch
    n = spec.T * spec.H
    x = torch.randn(n, device="cuda", dtype=torch.bfloat16)
    dst = torch.empty_like(x)
    acc = torch.empty((), device="cuda", dtype=torch.float32)
    res = {"workload": spec.name, "bytes": 2 * n}
    for name, fn, moved in (("copy", lambda: dst.copy_(x), 4 * n),
                            ("sum", lambda: torch.sum(x, dim=0, dtype=torch.float32, out=acc), 2 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        calls, t0 = 0, time.perf_counter()
        e0.record()
        while calls < 20 or time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            calls += 20
            torch.cuda.synchronize()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        res[name] = {"calls": calls, "us": us, "GB/s": moved / (us * 1e-6) / 1e9,
                     "frac_of_8TBs": moved / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return res


def cpu_baseline(spec, inp, limit_s: float):
    """Time the fp64 oracle on the host: the whole forward (gate, softmax, top-k,
    losses, dispatch, expert FFN, combine) over all T tokens when a probe
    predicts it fits in limit_s seconds; otherwise routing and dispatch over
    all T tokens plus the expert FFN and combine on a contiguous token prefix
    sized to limit_s, scaled linearly to T (the FFN is per token), and the
    sample says so."""
    import numpy as np
    import oracle as om
    t0 = time.perf_counter()
    lg = om.logits(spec, inp["x"], inp["Wg"], inp["bg"])
    if spec.ec_group:
        r = om.expert_choice(spec, lg, spec.ec_group)
        kept_mask = r["rowof"] >= 0
    else:
        r = om.route(spec, lg)
        dsp = om.dispatch(spec, r["topk_idx"])
        kept_mask = dsp["pos"] >= 0
    t_route = time.perf_counter() - t0

    def ffn(n):
        t1 = time.perf_counter()
        if spec.ec_group:
            om.ec_forward_tokens(spec, inp["x"], r["rowof"], r["probs"], inp["W1"],
                                 inp.get("b1"), inp["W2"], inp.get("b2"), np.arange(n))
        else:
            om.forward_tokens(spec, inp["x"], r["topk_idx"], r["topk_w"], dsp["pos"], inp["W1"],
                              inp.get("b1"), inp["W2"], inp.get("b2"), np.arange(n))
        return time.perf_counter() - t1

    threads = om.num_threads()
    n0 = min(spec.T, max(threads, 8))
    t_probe = ffn(n0)
    est = t_probe * spec.T / n0
    if est <= limit_s:
        n = spec.T
    else:
        n = int(min(spec.T, max(n0, n0 * max(limit_s - t_route, 1.0) / max(t_probe, 1e-6))))
    t_ffn = ffn(n) if n > n0 else t_probe
    total = t_route + t_ffn * spec.T / n
    kept = int(kept_mask[:n].sum())                          # kept pairs of the timed tokens
    flops = 2.0 * spec.T * spec.H * spec.E + 4.0 * spec.H * spec.F * kept
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    route_what = ("gate/softmax/expert choice" if spec.ec_group
                  else "gate/softmax/top-k/losses/dispatch")
    if n == spec.T:
        sample = (f"fp64 C oracle, {threads} OpenMP threads: the whole forward of all "
                  f"{spec.T} tokens ({route_what} {t_route:.2f} s, expert FFN and combine "
                  f"{t_ffn:.2f} s), no scaling")
    else:
        sample = (f"fp64 C oracle, {threads} OpenMP threads: {route_what} over all {spec.T} "
                  f"tokens ({t_route:.2f} s) + expert FFN and combine on tokens 0..{n - 1} "
                  f"({t_ffn:.2f} s), FFN time scaled linearly to {spec.T} tokens "
                  f"(the whole forward was estimated at {est:.0f} s)")
    return {"value": spec.T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": cpu, "gflops": flops / (t_route + t_ffn) / 1e9, "seconds": t_route + t_ffn,
            "scaled": n != spec.T, "sample": sample}


def _dense_coords(p, real_mt, Nt, SBN):
    """Tile (mt, nt) at position p of the expert GEMMs' XCD-aware tile order
    (the library's dense_coords, restated for the byte count below)."""
    SBM = 256 // SBN
    if Nt % SBN:
        return p // Nt, p % Nt
    F = real_mt // SBM
    nfull = F * SBM * Nt
    if p < nfull:
        sb, q = p >> 8, p & 255
        x, j = q & 7, q >> 3
        nsbn = Nt // SBN
        s8 = (x + sb) & 7
        xm, xn = s8 % (SBM // 8), s8 // (SBM // 8)
        return (sb // nsbn) * SBM + xm * 8 + (j & 7), (sb % nsbn) * SBN + xn * 4 + (j >> 3)
    q, rem = p - nfull, real_mt - F * SBM
    if Nt % 8 == 0:
        x, j = q & 7, q >> 3
        return F * SBM + j % rem, 8 * (j // rem) + x
    return F * SBM + q // Nt, q % Nt


def combine_cut_extra_bytes(T, k, E, H, F, cf, counts_kept, ncu):
    """Bytes the combine of the top-k bf16 forward reads beyond a plain combine:
    the second GEMM's cut tiles reach it as S fp32 K-slice partials instead of
    bf16 y rows.  The plan follows the library: row tile height from the mean
    expert load, the ragged last round of R = row tiles x column tiles cut into
    S = min(min(ncu, 256) / tail, k-tiles / stages) slices when S >= 2."""
    cap = T if cf <= 0 else min(math.ceil(cf * T * k / E), T)
    avg = min((T * k + E - 1) // E, cap)
    bm = 64 if avg <= 32 else 128 if avg <= 128 else 256
    bk, ns = (64, 2) if bm == 256 else (32, 4)
    nk = (F + bk - 1) // bk
    Nt = (H + 255) // 256
    SBN = 16 if Nt % 16 == 0 else 8 if Nt % 8 == 0 else 4
    tiles = [(int(n) + bm - 1) // bm for n in counts_kept]
    real_mt = sum(tiles)
    R = real_mt * Nt
    tail = R % ncu
    if tail == 0:
        return 0
    S = min(min(ncu, 256) // tail, nk // ns)
    if S < 2:
        return 0
    first = [sum(tiles[:e]) for e in range(E)]          # row tiles before expert e
    extra = 0
    for p in range(R - tail, R):
        mt, nt = _dense_coords(p, real_mt, Nt, SBN)
        e = max(i for i in range(E) if first[i] <= mt and tiles[i] > 0)
        rows = min(bm, int(counts_kept[e]) - (mt - first[e]) * bm)
        cols = min(256, H - 256 * nt)
        extra += rows * cols * (4 * S - 2)
    return extra


def routing_stats(E, counts, offsets, cap, T, k):
    """Per-expert load before and after capacity, and what capacity dropped."""
    import numpy as np
    counts = np.asarray(counts, np.int64)
    kept = np.diff(np.asarray(offsets, np.int64))
    return {"load_max": int(counts.max()), "load_min": int(counts.min()),
            "kept_max": int(kept.max()), "kept_min": int(kept.min()),
            "experts_empty": int((counts == 0).sum()), "capacity": int(cap),
            "dropped_pairs": int(T * k - kept.sum()),
            "drop_fraction": float((T * k - kept.sum()) / (T * k))}


def _token_choice_calls(moe, prob, d, ws, out, losses, idx, tw, counts, offsets, pos, row_token,
                        xp, h, y):
    return {
        "forward": lambda: moe.moe_forward(prob, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"],
                                           d["W2"], d["b2"], out, losses, ws),
        "route": lambda: moe.moe_route(prob, d["x"], d["Wg"], d["bg"], None, idx, tw, counts,
                                       losses, ws),
        "permute": lambda: moe.moe_permute(prob, d["x"], idx, offsets, pos, row_token, xp, ws),
        "expert_ffn": lambda: moe.moe_expert_ffn(prob, xp, offsets, d["W1"], d["b1"], d["W2"],
                                                 d["b2"], h, y, ws),
        "combine": lambda: moe.moe_combine(prob, y, pos, tw, out),
    }


def stage_timing(moe, torch, spec, prob, d, log_fn, min_iters=50, min_seconds=0.5):
    """Every ABI call timed alone with HIP events on the caller's stream: 10
    warm-ups, then at least `min_iters` iterations and `min_seconds`; warm
    (back-to-back) and cold (a 512 MiB buffer written before every iteration,
    which flushes the 256 MB last-level cache).  Returns ms quantiles and the
    kept-row count A."""
    import numpy as np
    T, H, E, k, F = spec.T, spec.H, spec.E, spec.k, spec.F
    sd = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    cu = "cuda"
    ws = torch.empty(moe.moe_workspace_bytes(prob), dtype=torch.uint8, device=cu)
    out = torch.empty(T, H, dtype=sd, device=cu)
    losses = torch.empty(2, dtype=torch.float32, device=cu)
    idx = torch.empty(T, k, dtype=torch.int32, device=cu)
    tw = torch.empty(T, k, dtype=torch.float32, device=cu)
    counts = torch.empty(E, dtype=torch.int32, device=cu)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=cu)
    pos = torch.empty(T, k, dtype=torch.int32, device=cu)
    row_token = torch.empty(T * k, dtype=torch.int32, device=cu)
    xp = torch.empty(T * k, H, dtype=sd, device=cu)
    h = torch.empty(T * k, F, dtype=sd, device=cu)
    y = torch.empty(T * k, H, dtype=sd, device=cu)
    if spec.ec_group:
        # expert choice: the whole layer and its routing call
        g = spec.ec_group
        C = moe.moe_ec_capacity(prob, g)
        ws = torch.empty(moe.moe_ec_workspace_bytes(prob, g), dtype=torch.uint8, device=cu)
        probs = torch.empty(T, E, dtype=torch.float32, device=cu)
        rowof = torch.empty(T, E, dtype=torch.int32, device=cu)
        sel = torch.empty(E * (T // g) * C, dtype=torch.int32, device=cu)
        calls = {
            "forward": lambda: moe.moe_forward_expert_choice(
                prob, g, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"], out, ws),
            "route": lambda: moe.moe_route_expert_choice(prob, g, d["x"], d["Wg"], d["bg"], None,
                                                         probs, sel, rowof, offsets, ws),
        }
        A = E * (T // g) * C
    else:
        calls = _token_choice_calls(moe, prob, d, ws, out, losses, idx, tw, counts, offsets, pos,
                                    row_token, xp, h, y)
        for name in ("route", "permute", "expert_ffn", "combine"):   # inputs of later stages
            calls[name]()
        torch.cuda.synchronize()
        A = int(offsets[-1].item())
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=cu)
    res = {}
    for name, fn in calls.items():
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        est = (time.perf_counter() - t1) / 3
        n = max(min_iters, int(min_seconds / max(est, 1e-6)) + 1)
        row = {}
        for mode in ("warm", "cold"):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
            for a, b in evs:
                if mode == "cold":
                    flush.fill_(1)
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            ms = np.array([a.elapsed_time(b) for a, b in evs])
            row[mode] = {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                         "p90": float(np.percentile(ms, 90)), "n": n}
        res[name] = row
        log_fn(f"[bench] {name}: warm {row['warm']['median']:.4f} ms, cold {row['cold']['median']:.4f} ms")
    del flush
    return res, A


TRAIN_METRIC = "MoE layer training step (forward + backward) tokens/s on 1 MI355X"
G_AUX, G_Z = 0.01, 0.001


def train_bench(args, moe, torch, spec, inp, d, prob):
    """A training step: moe_forward_train then moe_backward for a fixed seeded
    upstream gradient; value = T / step time.  The roofline entry is the
    backward's dominant GEMM launch against the bf16 MFMA peak, timed by the
    library's own stage events."""
    import numpy as np
    import workloads as W
    T, H, E, k, F = spec.T, spec.H, spec.E, spec.k, spec.F
    cu = "cuda"
    ws = torch.empty(moe.moe_train_workspace_bytes(prob), dtype=torch.uint8, device=cu)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=cu)
    losses = torch.empty(2, dtype=torch.float32, device=cu)
    dout = torch.from_numpy(W.synthetic_rows(spec, T, tid=98).view(np.int16)).to(cu).view(
        torch.bfloat16)
    f32 = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=cu)
    dx = torch.empty(T, H, dtype=torch.bfloat16, device=cu)
    dWg, dW1, dW2 = f32(H, E), f32(E, H, F), f32(E, F, H)
    dbg = f32(E) if d["bg"] is not None else None
    db1 = f32(E, F) if d["b1"] is not None else None
    db2 = f32(E, H) if d["b2"] is not None else None
    evs = [moe.StageEvents(moe.MOE_BACKWARD_EVENTS) for _ in range(args.steps)]
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]

    def step(i=None):
        if i is not None:
            fev[i][0].record()
        moe.moe_forward_train(prob, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"],
                              out, losses, ws)
        if i is not None:
            fev[i][1].record()
        moe.moe_backward(prob, d["x"], d["Wg"], d["W1"], d["W2"], dout, G_AUX, G_Z, dx, dWg, dW1,
                         dW2, ws, dbg=dbg, db1=db1, db2=db2,
                         events=evs[i] if i is not None else None)

    log(f"[bench] train warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} training steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in fev]))
    bst = np.array([e.stage_ms() for e in evs]).mean(axis=0)
    sm = {n: float(v) for n, v in zip(moe.BACKWARD_STAGE_NAMES, bst)}
    A = T * k                    # kept rows (the training workloads drop nothing)
    gemm_flops = 2.0 * A * H * F
    gemms = ("dgrad_da", "dgrad_dxe", "wgrad_w2", "wgrad_w1")
    dom = max(gemms, key=lambda n: sm[n])
    achieved = gemm_flops / (sm[dom] * 1e-3) / 1e12
    bwd_ms = float(sum(bst))
    res = {
        "metric": TRAIN_METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded; random-init weights; seeded upstream gradient)",
        "config": {"workload": spec.name, "T": T, "H": H, "E": E, "k": k, "F": F,
                   "capacity_factor": spec.cf, "activation": spec.act,
                   "g_aux": G_AUX, "g_z": G_Z},
        "roofline": {"bound": "mfma", "kernel": f"bwd_{dom}", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None},
        "forward_train_ms": fwd_ms,
        "backward_ms": bwd_ms,
        "backward_stage_ms": sm,
        "train_tflops": 6.0 * gemm_flops / ((fwd_ms + bwd_ms) * 1e-3) / 1e12,
        "backward_gemm_tflops": 4.0 * gemm_flops / (sum(sm[n] for n in gemms) * 1e-3) / 1e12,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle's backward on a bounded sample")
        res["cpu_baseline"] = cpu_train_baseline(spec, inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def cpu_train_baseline(spec, inp, target_s: float):
    """The fp64 oracle's forward and backward (all gradients) on the first n
    tokens taken as a problem of their own, n sized to about target_s, scaled
    linearly to T (the work is per token)."""
    import oracle as om
    import workloads as W

    def run(n):
        sub = spec.replace(T=n)
        si = dict(inp)
        si["x"] = inp["x"][:n]
        dout = W.synthetic_rows(sub, n, tid=98)
        t1 = time.perf_counter()
        om.backward(sub, si, dout, G_AUX, G_Z)
        return time.perf_counter() - t1

    threads = om.num_threads()
    n0 = min(spec.T, 2 * threads)
    t_probe = run(n0)
    n = int(min(spec.T, max(n0, n0 * target_s / max(t_probe, 1e-6))))
    t = run(n) if n > n0 else t_probe
    return {"value": n / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"fp64 C oracle backward (recomputing the forward), {threads} OpenMP "
                       f"threads, on tokens 0..{n - 1} as a problem of their own ({t:.2f} s), "
                       f"rate scaled linearly to {spec.T} tokens")}


def main():
    args = parse()
    if args.summarize_pmc:
        import workloads as W
        out, lines = summarize_pmc(*args.summarize_pmc, W.CONFIGS[args.config].name,
                                   args.calibrate_copy or 256)
        with open(traffic_path(W.CONFIGS[args.config].name), "w") as fh:
            json.dump(out, fh, indent=1)
        print("\n".join(lines))
        print(f"fetch factor {out['fetch_factor']:.4f}, write factor {out['write_factor']:.4f} "
              f"(calibration: {out['calibration_kernel']})")
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_mixture_experts_21_amd as moe
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    spec = W.CONFIGS[args.config]
    if args.vendor_gemm > 0:
        print(json.dumps(vendor_gemm(spec, args.vendor_gemm)), flush=True)
        return
    if args.vendor_stream > 0:
        print(json.dumps(vendor_stream(spec, args.vendor_stream)), flush=True)
        return
    moe.lib()

    T, H, E, k, F = spec.T, spec.H, spec.E, spec.k, spec.F
    log(f"[bench] generating {spec.name}")
    t0 = time.perf_counter()
    inp = W.generate(spec)
    log(f"[bench] inputs drawn in {time.perf_counter() - t0:.1f} s")

    sd = torch.bfloat16 if spec.dtype == "bf16" else torch.float32

    def dev(a):
        if a is None:
            return None
        if spec.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {kk: dev(v) for kk, v in inp.items()}
    prob = moe.Problem.from_spec(spec)
    if args.train:
        train_bench(args, moe, torch, spec, inp, d, prob)
        return
    g = spec.ec_group
    ws_bytes = moe.moe_ec_workspace_bytes(prob, g) if g else moe.moe_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(T, H, dtype=sd, device="cuda")
    losses = torch.empty(2, dtype=torch.float32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    rowof = torch.empty(T, E, dtype=torch.int32, device="cuda") if g else None
    # Every recorded event adds a few microseconds between two kernels, so the
    # stage breakdown comes from its own instrumented pass, and the timed
    # region records only the two events around the dominant GEMM launch.
    evs = [moe.StageEvents() for _ in range(args.steps)]

    def step(ev=None):
        if g:       # expert choice: every expert takes C tokens of each group
            moe.moe_forward_expert_choice(prob, g, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"],
                                          d["W2"], d["b2"], out, ws, rowof=rowof, events=ev)
        else:
            moe.moe_forward(prob, d["x"], d["Wg"], d["bg"], d["W1"], d["b1"], d["W2"], d["b2"],
                            out, losses, ws, counts=counts, offsets=offsets, events=ev)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] stage breakdown over {args.steps} instrumented steps")
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    stage_pass = np.array([ev.stage_ms() for ev in evs])     # [steps][stages]
    names_ = moe.STAGE_NAMES
    up_i, down_i = names_.index("ffn_up"), names_.index("ffn_down")
    dom_i = up_i if stage_pass[:, up_i].mean() >= stage_pass[:, down_i].mean() else down_i
    tevs = [moe.StageEvents(points=(dom_i, dom_i + 1)) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(tevs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    # the dominant GEMM launch, timed inside the timed region on the library's stream
    dom_ms_timed = float(np.mean([ev.elapsed_ms(dom_i, dom_i + 1) for ev in tevs]))

    graph = None
    if not args.no_graph:
        # The same forward captured once into a HIP graph and replayed K times:
        # what a serving loop that replays its layer pays without per-launch
        # host overhead.  `value` stays the eager rate.
        log(f"[bench] timing {args.steps} graph replays")
        ref_out = out.clone()
        gr = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(gr):
            step()
        gr.replay()
        torch.cuda.synchronize()
        same = bool(torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                                ref_out.view(torch.int16) if out.dtype == torch.bfloat16
                                else ref_out))
        t0 = time.perf_counter()
        for _ in range(args.steps):
            gr.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph = {"ms_per_step": gms, "tokens_per_s": T / (gms * 1e-3),
                 "output_equals_eager": same}
        del gr

    abi, A_abi = None, None
    if not args.no_abi_timing:
        log("[bench] timing each ABI call alone (warm and cold)")
        abi, A_abi = stage_timing(moe, torch, spec, prob, d, log)
    stage_mean = stage_pass.mean(axis=0)
    if g:
        A = E * (T // g) * moe.moe_ec_capacity(prob, g)
    else:
        A = int(offsets[-1].item())
    names = moe.STAGE_NAMES
    sm = {n: float(v) for n, v in zip(names, stage_mean)}
    gemm_flops = 2.0 * A * H * F                              # per GEMM launch
    ffn_ms = sm["ffn_up"] + sm["ffn_up_fixup"] + sm["ffn_down"] + sm["ffn_down_fixup"]
    ffn_tflops = 2 * gemm_flops / (ffn_ms * 1e-3) / 1e12
    dom = names_[dom_i]
    s = spec.elem_bytes
    # Each GEMM launch reads the weights of the experts that got rows and the
    # A rows of its input, and writes A rows: with few rows per expert that
    # stream, not the MFMAs, bounds it.
    active = E if g else int(np.sum(np.diff(offsets.cpu().numpy()) > 0))
    gemm_bytes = active * H * F * s + A * (H + F) * s
    bound = "mfma" if gemm_flops / (PEAK_BF16_TFLOPS * 1e12) >= gemm_bytes / (PEAK_HBM_GBS * 1e9) \
        else "hbm"
    if bound == "mfma":
        achieved, peak, unit = gemm_flops / (dom_ms_timed * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = gemm_bytes / (dom_ms_timed * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    nblk = (T + 15) // 16                                     # router blocks = dispatch chunks
    if g:
        alg_bytes = {
            # x and the gate in; fp32 logits, top-k scratch and partials out
            "route": T * H * s + H * E * s + T * E * 4 + T * k * 8 + nblk * (2 * E + 1) * 4,
            # logits in; probs, rowof and the selected tokens out
            "permute": 3 * T * E * 4 + A * 4,
            # selected rows in, rowof and probs in, token rows out
            "combine": A * H * s + T * E * 8 + T * H * s,
        }
    else:
        alg_bytes = {
            # x and the gate in; top-k ids and weights, per-block partials out
            "route": T * H * s + H * E * s + T * k * 8 + nblk * (2 * E + 1) * 4,
            # block histograms in, chunk bases out and back in, ids in, pos and
            # row_token out (the row gather is fused into ffn_up in moe_forward)
            "permute": 3 * nblk * E * 4 + T * k * 8 + A * 4,
            # kept expert rows in, slot rows and weights in, token rows out; the
            # second GEMM's cut tiles come in as fp32 K-slice partials
            "combine": A * H * s + T * k * 8 + T * H * s + (
                combine_cut_extra_bytes(T, k, E, H, F, spec.cf,
                                        np.diff(offsets.cpu().numpy()),
                                        torch.cuda.get_device_properties(0).multi_processor_count)
                if spec.dtype == "bf16" else 0),
        }
    hbm = {n: {"ms": sm[n], "GB/s": alg_bytes[n] / (sm[n] * 1e-3) / 1e9,
               "frac": alg_bytes[n] / (sm[n] * 1e-3) / 1e9 / PEAK_HBM_GBS} for n in alg_bytes}
    # calibrated FETCH + WRITE bytes of the stage's kernels from profiles/, when
    # they were taken on these sources and this workload
    # (each entry: the stage's kernels; a tuple names alternatives, the first
    # one measured counts: the combine that finishes the cut tiles, or the plain one)
    stage_kernels = {"route": ("route_bf16",), "permute": ("scan_columns", "chunk_rank"),
                     "combine": (("combine_rows_cut", "combine_rows"),)}
    for n, ks in stage_kernels.items():
        tr = [next((v for v in (traffic_for(a, spec.name) for a in kk) if v is not None), None)
              if isinstance(kk, tuple) else traffic_for(kk, spec.name) for kk in ks]
        if n in hbm:
            hbm[n]["traffic"] = None if g or any(v is None for v in tr) else sum(tr)
    kern = "ffn_gemm_bf16_up" if dom == "ffn_up" else "ffn_gemm_bf16_down"
    res = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded; random-init weights)",
        "config": {"workload": spec.name, "T": T, "H": H, "E": E, "k": k, "F": F,
                   "capacity_factor": spec.cf, "activation": spec.act, "kept_rows": A,
                   "routing": f"expert choice, groups of {g}" if g else f"top-{k}"},
        "roofline": {"bound": bound, "kernel": kern, "achieved": achieved, "peak": peak,
                     "unit": unit, "frac": achieved / peak,
                     "traffic": traffic_for(kern, spec.name)},
        "ffn_tflops": ffn_tflops,
        "ffn_frac_of_bf16_peak": ffn_tflops / PEAK_BF16_TFLOPS,
        "graph": graph,
        "dominant_kernel_ms": dom_ms_timed,
        "stage_ms": sm,
        "hbm_stages": hbm,
        "abi_ms": abi,
        "abi_ffn_tflops": None if abi is None or g else {
            m: 4.0 * H * F * A_abi / (abi["expert_ffn"][m]["median"] * 1e-3) / 1e12
            for m in ("warm", "cold")},
        "abi_hbm_frac_cold": None if abi is None or g else {
            "route": (T * H * s + H * E * s + T * k * 8) / (abi["route"]["cold"]["median"] * 1e-3)
                     / 1e9 / PEAK_HBM_GBS,
            "permute": (T * k * 4 + T * H * s + A_abi * H * s + 2 * A_abi * 4)
                       / (abi["permute"]["cold"]["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "combine": (A_abi * H * s + T * k * 8 + T * H * s)
                       / (abi["combine"]["cold"]["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
        },
        "losses": None if g else [float(v) for v in losses.cpu().numpy()],
        "routing_stats": routing_stats(E, counts.cpu().numpy(), offsets.cpu().numpy(),
                                 moe.moe_capacity(prob), T, k) if not g else {
            "rows_per_expert": A // E, "capacity_per_group": moe.moe_ec_capacity(prob, g),
            "tokens_taken_by_no_expert": int(((rowof >= 0).sum(dim=1) == 0).sum().item()),
            "tokens_taken_by_3_or_more": int(((rowof >= 0).sum(dim=1) >= 3).sum().item())},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(spec, inp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    # Context from the same machine, after the timed work: the vendor library's
    # batched GEMM on the expert shapes (balanced experts) and plain streams
    # over a buffer of x's size.  Not part of the layer or of its figures.
    if not args.no_vendor_reference and spec.dtype == "bf16" and T * k // E >= 256:
        log("[bench] vendor side references (torch.bmm, copy, sum)")
        res["vendor_reference"] = {"gemm": vendor_gemm(spec, 1.0),
                                   "stream": vendor_stream(spec, 0.5)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
