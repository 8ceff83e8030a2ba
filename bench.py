#!/usr/bin/env python3
"""Throughput of the CSA2 decode hot path on one MI355X.

One step = one pass of the whole path for one batch of synthetic input: the Full indexer scan
over every visible position, the block candidate pool and Top-K, every Reindex layer (re-score
the pool with its own query, Top-K) and sparse attention for every attention layer (FP4 main
KV rows of the layer's index set merged with its FP8 window).  Reuse layers run attention on
their leader's index set.  Default workload: batch 1 decode over a 1M-entry context
(Full + 4 Reindex + 15 Reuse layers, 16 attention heads).  Workloads without a Full layer
(caller pools) time the Reindex layers and attention.

Inputs are resident in HBM before timing.  The context (indexer K and main KV) is replicated
``--replicas`` times at distinct addresses and steps rotate over the replicas, so the 256 MB
Infinity Cache cannot serve the 128 MiB indexer-K stream from one step to the next.  Every
kernel is launched directly on one stream that the host keeps ahead of the GPU (measured as
fast as replaying one HIP graph per step, and faster than a graph for the part after the
scan); the first kernel of each timed step (the scan; the Reindex stage without a Full layer)
sits between two timing events, which bracket that launch (the scan's duration is the
roofline figure).

Prints one JSON line (metric, value in queries/s, roofline of the scan kernel, CPU oracle
baseline) on stdout; a per-stage breakdown goes to stderr.

``--kernel quantize_kv`` instead times the FP4 main-KV quantiser on its own (2^20 latent rows
per launch by default, ``--rows``) and prints its own JSON line (rows/s, HBM roofline).

``--summarize-pmc FETCH_DIR WRITE_DIR`` turns two rocprofv3 counter runs of this script
(``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, each with ``--calibrate-copy``) into the
traffic summary that later runs report, and exits.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/s at 1M ctx (Full+Reindex+attn); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
SCAN_SOURCES = ("hierarchical_kv_indexer_amd/csrc/scan.hip", "hierarchical_kv_indexer_amd/csrc/common.hpp")
PMC_FILE = os.path.join(ROOT, "profiles", "k_idx_scan_decode_1m_pmc.json")
KERNEL_FILE = os.path.join(ROOT, "profiles", "decode_1m_kernels.json")
COPY_BYTES = 256 << 20          # plain device copy that calibrates the HBM byte counters
IDX_Q_BYTES = 32 * 128 * 2      # one indexer query (bf16)
IDX_W_BYTES = 32 * 4            # its head weights
KV_ROW_BYTES = 256 + 32         # FP4 codes + E4M3 scales of one main-KV entry


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_source_hash() -> str:
    h = hashlib.sha1()
    for p in SCAN_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def key_row_bytes(w) -> int:
    """Bytes of one indexer-K position: 128 E4M3 bytes, or 64 E2M1 code bytes + 8 E4M3 scales."""
    return 72 if w.idx_k_fp4 else 128


def scan_algorithmic_bytes(w) -> int:
    """Bytes one scan launch must move: every visible indexer-K row (128 B, or 72 B for FP4 keys)
    of every query (a prefill's queries share one context: its rows count once), plus each query's
    indexer query and head weights."""
    q = w.B * w.T
    if w.prefill_tokens:
        rows = w.B * int(w.n_visible().max())
    else:
        rows = int(w.n_visible().astype("int64").sum())
    return rows * key_row_bytes(w) + q * (IDX_Q_BYTES + IDX_W_BYTES)


def reindex_layer_bytes(w) -> int:
    """One Reindex layer, one query: the pool's K rows, the pool, Q, w and the Top-K written."""
    return w.pool_cap * (key_row_bytes(w) + 4) + IDX_Q_BYTES + IDX_W_BYTES + w.top_k * 4


def attention_layer_bytes(w) -> int:
    """One attention layer, one query: indices, gathered FP4 rows, window rows, q in, out."""
    return w.top_k * (4 + KV_ROW_BYTES) + w.swa_window * 512 + 2 * w.H * 512 * 2


def step_algorithmic_bytes(w) -> int:
    """Bytes one whole step must move, per stage (the accounting of the design notes)."""
    q = w.B * w.T
    b = 0
    if w.has_full:
        b += scan_algorithmic_bytes(w)
        b += q * (w.pool_cap * 4 if w.pool_blocks else 0)   # pool written
        b += q * w.top_k * 4                                 # Full Top-K written
    b += w.n_reindex * q * reindex_layer_bytes(w)
    b += w.L * q * attention_layer_bytes(w)
    return b


def traffic_from_profile():
    """HBM bytes per scan launch from the committed rocprofv3 counter summary, or None when the
    scan kernel's sources changed since the counters were taken."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha1") != scan_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_means(run_dir: str, counter: str):
    """Mean counter value per dispatch (KiB) for the scan kernel and the calibration copy."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    scan, copy = [], []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            v, name = float(r["Counter_Value"]), r.get("Kernel_Name", "")
            if "k_idx_scan" in name:
                scan.append(v)
            elif "copy" in name.lower():
                copy.append(v)
    if not scan or not copy:
        raise SystemExit(f"{counter}: found {len(scan)} scan and {len(copy)} copy dispatches")
    copy.sort()
    big = [c for c in copy if c >= 0.5 * copy[-1]]   # the calibration copies are the largest
    return sum(scan) / len(scan), sum(big) / len(big), len(scan), len(big)


def summarize_pmc(fetch_dir: str, write_dir: str) -> int:
    fs, fc, nfs, nfc = _counter_means(fetch_dir, "FETCH_SIZE")
    ws, wc, nws, nwc = _counter_means(write_dir, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    f_fetch, f_write = kib / fc, kib / wc              # counter KiB -> true KiB
    traffic = (fs * f_fetch + ws * f_write) * 1024.0
    out = {
        "kernel": "k_idx_scan", "workload": "decode_1m", "source_sha1": scan_source_hash(),
        "fetch_kib_per_launch": round(fs, 1), "write_kib_per_launch": round(ws, 1),
        "copy_bytes": COPY_BYTES, "copy_fetch_kib": round(fc, 1), "copy_write_kib": round(wc, 1),
        "fetch_scale": round(f_fetch, 4), "write_scale": round(f_write, 4),
        "hbm_bytes_per_launch": int(traffic),
        "dispatches": {"scan_fetch": nfs, "copy_fetch": nfc, "scan_write": nws, "copy_write": nwc},
    }
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def _median_rate(run_once, seconds: float, max_runs: int):
    """Median over 3 timed runs of the rate of run_once(); each run repeats it for about
    `seconds` / 3 (at least once, at most max_runs times)."""
    rates, n_total = [], 0
    for _ in range(3):
        n, t0 = 0, time.perf_counter()
        while True:
            run_once()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds / 3 or n >= max_runs:
                break
        rates.append(n / el)
        n_total += n
    rates.sort()
    return rates[1], n_total


def _oracle_threads():
    """Threads the oracle's numpy/BLAS work may use on this host: the CPUs this process may run on
    (the BLAS pool's own limit applies on top; see _blas_threads)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def cpu_baseline(w, inp, seconds: float):
    """The oracle, as it stands, on this host: the whole chain for query (0, 0), timed with its
    BLAS pool limited to 1 thread and then with every thread it may use (median of 3 runs each).
    Only the oracle's matrix products run on several threads; the rest of it (block scores,
    ranking, attention rows) is serial numpy.  `cores` is the thread count of the all-threads
    run."""
    from oracle import csa2 as O
    from threadpoolctl import threadpool_limits

    def once():
        O.query_chain(inp, w, 0, 0)

    threads = min(_oracle_threads(), _blas_threads())
    with threadpool_limits(limits=1):
        r1, n1 = _median_rate(once, seconds / 2, 20)
    with threadpool_limits(limits=threads):
        rn, nn = _median_rate(once, seconds / 2, 20)
    what = (f"Full scan of {w.N} positions, pool, Top-{w.top_k}, " if w.has_full else "caller pool, ")
    return {"value": rn, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": r1,
            "sample": f"the whole chain ({what}{w.n_reindex} Reindex layers, {w.L} attention layers) for one "
                      f"query of {w.name}; median of 3 runs at {threads} BLAS threads ({nn} chains) and at 1 "
                      f"thread ({n1} chains), {_oracle_threads()} CPUs available"}


def measure_copy_gbps(dev, stream, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Bytes read plus written per second by a plain device-to-device copy of nbytes (torch's copy
    kernel), timed with events on `stream`: the practical ceiling of a one-pass kernel here."""
    import torch
    src = torch.full((nbytes,), 1, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        dst.copy_(src)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            dst.copy_(src)
            b.record(stream)
        torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def kernel_duration_from_profile(kernel: str, workload: str):
    """Average duration (us) of `kernel` at `workload` from the committed rocprofv3 kernel-trace
    summary, or None when it is missing or the kernel's sources changed since it was taken."""
    try:
        with open(KERNEL_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha1") != scan_source_hash() or d.get("workload") != workload:
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("avg_us")


QUANT_ROW_BYTES = 512 * 2 + 256 + 32      # bf16 latent row in, E2M1 codes and E4M3 scales out


def bench_quantize_kv(args) -> int:
    """The FP4 main-KV quantiser alone: `rows` latent rows per launch (seeded normal rows with a
    few large channels, unit RMS as after RMSNorm), launches timed with events on their stream.
    Algorithmic bytes per launch: rows x (1024 read + 288 written)."""
    import numpy as np
    import torch

    import hierarchical_kv_indexer_amd as H
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H.lib()
    rows, R = args.rows, args.replicas
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    xs = []
    for _ in range(R):       # distinct inputs and outputs per replica (past the Infinity Cache)
        x = torch.randn((rows, 512), generator=g, device=dev, dtype=torch.float32)
        x[:, 7] *= 8.0
        xs.append(x.to(torch.bfloat16))
        del x
    codes = [torch.empty((rows, 256), dtype=torch.uint8, device=dev) for _ in range(R)]
    scales = [torch.empty((rows, 32), dtype=torch.uint8, device=dev) for _ in range(R)]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        if args.calibrate_copy:
            src_buf = torch.full((COPY_BYTES,), 1, dtype=torch.uint8, device=dev)
            dst_buf = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
            for _ in range(3):
                dst_buf.copy_(src_buf)
            torch.cuda.synchronize()
            del src_buf, dst_buf
        for i in range(args.warmup):
            r = i % R
            H.csa2_quantize_kv_fp4(xs[r], rows, codes[r], scales[r])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            r = i % R
            ev[i][0].record(stream)
            H.csa2_quantize_kv_fp4(xs[r], rows, codes[r], scales[r])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    wall = t1 - t0
    nbytes = rows * QUANT_ROW_BYTES
    achieved = nbytes / (launch_ms * 1e-3) / 1e9
    log(f"[bench] quantize_kv: {args.steps} launches of {rows} rows, {launch_ms * 1e3:.2f} us per launch, "
        f"{achieved:.0f} GB/s algorithmic")
    res = {
        "metric": "FP4 main-KV quantise rows/s (rotated bf16 latent -> E2M1 codes + E4M3 per-16 scales)",
        "value": round(args.steps * rows / wall, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"quantize_kv_{rows}", "rows": rows, "row_bytes": QUANT_ROW_BYTES,
                   "replicas": R},
        "roofline": {"bound": "hbm", "kernel": "k_quantize_kv", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(launch_ms * 1e3, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import formats as F
        n_cpu = 16384
        bits = xs[0][:n_cpu].view(torch.int16).cpu().numpy().view(np.uint16)
        t = time.perf_counter()
        n = 0
        while time.perf_counter() - t < min(args.cpu_seconds, 10.0) or n == 0:
            F.kv_quantize_rows(bits)
            n += 1
        el = time.perf_counter() - t
        res["cpu_baseline"] = {"value": round(n * n_cpu / el, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} runs of the oracle quantiser over {n_cpu} rows, {el:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / fp16 matrix peak


def bench_encoder(args, w) -> int:
    """One chunk of an encoder prefill (csa2_encoder_chunk): the last `T` tokens of a prompt of
    `prompt` tokens through `G` groups of one Full and `layers`-1 Reuse layers.  The caches
    already hold every earlier entry; each step appends the chunk's entries again (the same
    bytes) and recomputes the chunk.  The roofline is that of the Full scan (the multi-query
    k_idx_scan_mq, bf16 MFMA), timed on its own through csa2_index_scan with the arguments the
    chunk entry passes it: FLOPs per launch = 8192 x the visible entries of every token."""
    import numpy as np
    import torch

    import hierarchical_kv_indexer_amd as H
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H.lib()
    t_gen = time.perf_counter()
    inp = workloads.make_encoder_chunk(w)
    log(f"[bench] generated {w.name} inputs in {time.perf_counter() - t_gen:.1f} s")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    G_, L, B, T, Hh, K, m, p0 = w.G, w.layers, w.B, w.T, w.H, w.top_k, w.m, w.p0
    d = {k: up(v) for k, v in inp.items()}
    inp = None
    swa_rows = w.hist(p0) + T
    out = torch.empty((G_, L, B, T, Hh, 512), dtype=torch.int16, device=dev)
    ws_bytes = H.csa2_encoder_chunk_workspace(B, T, w.k_rows, L, Hh, K, w.swa_window)
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(512)
    stream = torch.cuda.Stream()

    def step():
        H.csa2_encoder_chunk(G_, L, d["new_idx_k"], d["new_latent"], d["idx_k"], d["kv_codes"], d["kv_scales"],
                             w.k_rows, d["idx_q"], d["head_w"], d["q"], d["swa"], swa_rows, B, T, p0, m, Hh, K,
                             w.swa_window, scale, out, None, ws, ws_bytes, stream)

    n_after = (p0 + T) // m
    nv = np.array([(p0 + t + 1) // m for t in range(T)], np.int32)
    nv_dev = up(np.broadcast_to(nv, (B, T)).copy())
    fws_bytes = H.csa2_index_stages_workspace(B, T, n_after, 8, 0, K)
    fws = torch.empty((fws_bytes,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # the Full scan of group 0 on its own, as the chunk entry launches it
        n_scan = max(3, min(20, args.steps))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_scan)]
        for i in range(n_scan):
            ev[i][0].record(stream)
            H.csa2_index_scan(d["idx_k"][0], None, w.k_rows, d["idx_q"][0], d["head_w"][0], nv_dev, B, T, n_after,
                              8, 0, K, fws, fws_bytes, stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
    wall = t1 - t0
    scan_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = 8192.0 * B * float(nv.astype(np.int64).sum())
    achieved = flops / (scan_ms * 1e-3) / 1e12
    step_flops = G_ * flops + G_ * L * B * T * Hh * 4.0 * 512 * (K + w.swa_window)
    log(f"[bench] {args.steps} steps in {wall:.3f} s: {wall * 1e3 / args.steps:.3f} ms/step; Full scan "
        f"{scan_ms * 1e3:.1f} us ({achieved:.0f} TFLOP/s bf16); whole chunk {step_flops * args.steps / wall / 1e12:.0f} "
        f"TFLOP/s")
    res = {
        "metric": "encoder prefill tokens/s (chunk at the end of a long prompt, Full + Reuse groups)",
        "value": round(args.steps * B * T / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "prompt_tokens": w.prompt, "chunk_tokens": T, "m": m,
                   "visible_entries_last_token": int(nv[-1]), "groups": G_, "layers_per_group": L,
                   "attention_heads": Hh, "indexer_heads": 32, "indexer_dim": 128, "top_k": K,
                   "swa_window": w.swa_window, "step_flops": step_flops},
        "roofline": {"bound": "mfma", "kernel": "k_idx_scan_mq", "achieved": round(achieved, 1),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flops_per_launch": flops, "avg_launch_us": round(scan_ms * 1e3, 3)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_encoder(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


KERNEL_NAMES = ("k_idx_scan", "k_pool_chunks", "k_pool", "k_ri_score", "k_topk", "k_sparse_attn",
                "k_attn_combine")


def summarize_trace(trace_dir: str, workload: str, steps: int) -> int:
    """Turns a rocprofv3 --kernel-trace --stats run of this script into the kernel-duration summary
    later runs report (profiles/decode_1m_kernels.json): per kernel of the chain, its calls per
    step and average duration, keyed to the scan's source hash."""
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    kernels = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            name = r.get("Name", "")
            short = next((k for k in KERNEL_NAMES if k + "<" in name or k + "(" in name or name.endswith(k)), None)
            if short is None:
                continue
            calls, avg = int(r["Calls"]), float(r["AverageNs"])
            if short in kernels:                   # template variants of one kernel: merge
                c0, a0 = kernels[short]["calls"], kernels[short]["avg_us"] * 1e3
                avg = (a0 * c0 + avg * calls) / (c0 + calls)
                calls += c0
            kernels[short] = {"calls": calls, "avg_us": round(avg / 1e3, 3)}
    out = {"workload": workload, "source_sha1": scan_source_hash(), "profiled_steps": steps,
           "kernels": kernels, "stats_file": os.path.relpath(files[0], trace_dir)}
    os.makedirs(os.path.dirname(KERNEL_FILE), exist_ok=True)
    with open(KERNEL_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


def cpu_baseline_encoder(w, seconds: float):
    """The oracle, as it stands, on this host: the measured chunk's tokens through the first group
    (Full layer over every visible entry, then the group's attention layers), one token after the
    other as one-token chunks (each appends the entries it completes); the rate is divided by the
    number of groups.  Inputs come from the same generator (group 0's draws)."""
    import dataclasses

    import workloads
    from oracle import csa2 as O
    cores = min(_oracle_threads(), _blas_threads())
    inp = workloads.make_encoder_chunk(dataclasses.replace(w, G=1))
    h, n0 = w.hist(w.p0), w.p0 // w.m
    n = 0
    t0 = time.perf_counter()
    while True:
        p = w.p0 + n
        e0, e1 = p // w.m - n0, (p + 1) // w.m - n0          # entries this token completes
        hp = w.hist(p)
        O.encoder_chunk(inp["idx_k"], inp["kv_codes"], inp["kv_scales"], inp["new_idx_k"][:, :, e0:e1],
                        inp["new_latent"][:, :, e0:e1], inp["idx_q"][:, :, n:n + 1], inp["head_w"][:, :, n:n + 1],
                        inp["q"][:, :, :, n:n + 1], inp["swa"][:, :, :, h + n - hp:h + n + 1], p, w.m, w.top_k,
                        w.swa_window)
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= 2) or n >= min(w.T, 50):
            break
    return {"value": n / el / w.G, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} tokens of the chunk through 1 of {w.G} groups (Full layer over "
                      f"{(w.p0 + 1) // w.m}+ entries, {w.layers} attention layers), {el:.1f} s; rate / {w.G}"}


def study_hsi_recall(args) -> int:
    """Recall study of the hierarchical indexer: on planted-needle contexts of 64K, 256K and 1M
    positions (workloads.make_recall_context), the Full layer's pool of P blocks ranked by each
    block score (max / sum / top-2 mean) and a Reindex layer's Top-512 inside that pool.  Reports,
    per (context, P, block score): the share of each needle family in the Full Top-512 and in the
    Reindex Top-512, and the share of the Reindex layer's dense Top-512 (over every position, no
    pool) that its pool-restricted Top-512 keeps.  A second sweep repeats the max block score with
    Reindex queries correlated with the Full query (rho).  Prints one JSON line per configuration."""
    import numpy as np
    import torch

    import hierarchical_kv_indexer_amd as H
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H.lib()

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    K = 512
    modes = {0: "max", 1: "sum", 2: "top2"}

    def sweep(N, seed, pools, block_scores, rho=None):
        ctx = workloads.make_recall_context(N, seed, rho=rho)
        k, q, hw, nv = up(ctx["idx_k"]), up(ctx["idx_q"]), up(ctx["head_w"]), up(ctx["n_visible"])
        rq, rw = up(ctx["ri_q"]), up(ctx["ri_w"])
        # the Reindex layer's dense Top-512 (no pool)
        wsd = H.csa2_index_full_workspace(1, 1, N, 8, 0, K)
        ws = torch.empty((wsd,), dtype=torch.uint8, device=dev)
        dense = torch.empty((1, 1, K), dtype=torch.int32, device=dev)
        H.csa2_index_full(k, None, N, rq[0], rw[0], nv, 1, 1, N, 8, 0, K, None, None, dense, None, ws, wsd)
        dense_set = set(dense.cpu().numpy().reshape(-1).tolist()) - {-1}
        for P in pools:
            wsb = H.csa2_index_chain_workspace(1, 1, N, 8, P, K, 1)
            ws = torch.empty((wsb,), dtype=torch.uint8, device=dev)
            pool_pos = torch.empty((1, 1, P * 8), dtype=torch.int32, device=dev)
            pool_len = torch.empty((1, 1), dtype=torch.int32, device=dev)
            ftop = torch.empty((1, 1, K), dtype=torch.int32, device=dev)
            rtop = torch.empty((1, 1, 1, K), dtype=torch.int32, device=dev)
            for bs in block_scores:
                H.csa2_index_scan_blocks(k, None, N, q, hw, nv, 1, 1, N, 8, P, K, bs, ws, wsb)
                H.csa2_index_select_reindex(k, None, N, nv, 1, 1, N, 8, P, K, rq, rw, 1, pool_pos, pool_len, ftop,
                                            None, rtop, None, ws, wsb)
                torch.cuda.synchronize()
                f = ftop.cpu().numpy().reshape(-1)
                r = rtop.cpu().numpy().reshape(-1)
                row = {"context": N, "pool_blocks": P, "block_score": modes[bs]}
                if rho is not None:
                    row["rho"] = rho
                row.update({
                    "full_topk": {fam: round(float(np.isin(pos, f).mean()), 4) for fam, pos in ctx["families"].items()},
                    "reindex_topk": {fam: round(float(np.isin(pos, r).mean()), 4)
                                     for fam, pos in ctx["families"].items()},
                    "reindex_dense_kept": round(len(dense_set & set(r.tolist())) / max(1, len(dense_set)), 4)})
                print(json.dumps(row), flush=True)

    for N, seed in ((1 << 16, 4101), (1 << 18, 4102), (1 << 20, 4103)):
        sweep(N, seed, (256, 512, 1024, 2048), tuple(modes))
    for N, seed in ((1 << 16, 4101), (1 << 20, 4103)):
        for rho in (0.5, 0.8, 0.9, 0.95, 0.99, 1.0):
            sweep(N, seed, (512, 2048), (0,), rho)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_1m")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--graph", action="store_true",
                    help="replay everything after the first stage from a HIP graph (measured slower here)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-to-device copy measurement")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for the HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the kernel-duration summary of a rocprofv3 --stats run of this script "
                         "(--workload and --steps as in that run)")
    ap.add_argument("--kernel", choices=("chain", "quantize_kv"), default="chain",
                    help="quantize_kv: time the FP4 main-KV quantiser alone")
    ap.add_argument("--rows", type=int, default=1 << 20, help="latent rows per quantiser launch")
    ap.add_argument("--study", choices=("hsi_recall",), default=None,
                    help="hsi_recall: recall of planted needles under block-score variants and pool sizes")
    args = ap.parse_args()

    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.workload, args.steps)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the sharding plan is written up with the design notes).", file=sys.stderr)
        return 2

    if args.kernel == "quantize_kv":
        return bench_quantize_kv(args)
    if args.study == "hsi_recall":
        return study_hsi_recall(args)
    import workloads
    if args.workload in workloads.ENCODER_WORKLOADS:
        return bench_encoder(args, workloads.ENCODER_WORKLOADS[args.workload])

    import numpy as np
    import torch

    import hierarchical_kv_indexer_amd as H
    import workloads

    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    H.lib()
    t_gen = time.perf_counter()
    inp = workloads.make_inputs(w)
    log(f"[bench] generated {w.name} inputs in {time.perf_counter() - t_gen:.1f} s")

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    B, T, N, K, L, Hh, R = w.B, w.T, w.N, w.top_k, w.L, w.H, args.replicas
    Q = B * T
    if w.idx_k_fp4:
        k_rep = [up(inp["idx_k_codes"]) for _ in range(R)]
        ks_rep = [up(inp["idx_k_scales"]) for _ in range(R)]
    else:
        k_rep = [up(inp["idx_k"]) for _ in range(R)]
        ks_rep = [None] * R
    codes_rep = [up(inp["kv_codes"]) for _ in range(R)]
    scales_rep = [up(inp["kv_scales"]) for _ in range(R)]
    idx_q, head_w, n_vis = up(inp["idx_q"]), up(inp["head_w"]), up(inp["n_visible"])
    ri_q, ri_w = up(inp["ri_q"]), up(inp["ri_w"])
    qa, swa, swa_end = up(inp["q"]), up(inp["swa"]), up(inp["swa_end"])
    S = w.n_sets
    sets = torch.full((S, B, T, K), -1, dtype=torch.int32, device=dev)
    if w.has_full:
        pool_pos = torch.empty((B, T, w.pool_cap), dtype=torch.int32, device=dev) if w.pool_blocks else None
        pool_len = torch.empty((B, T), dtype=torch.int32, device=dev) if w.pool_blocks else None
    else:
        pool_pos, pool_len = up(inp["pool_pos"]), up(inp["pool_len"])
    out = torch.empty((L, B, T, Hh, 512), dtype=torch.int16, device=dev)
    lse = torch.empty((L, B, T, Hh), dtype=torch.float32, device=dev)
    chain = w.has_full and w.pool_blocks > 0          # pool, Full Top-K and Reindex in one call
    if chain:
        ws_full_b = H.csa2_index_chain_workspace(B, T, N, w.block, w.pool_blocks, K, w.n_reindex)
    else:
        # csa2_index_full over every query at once (a workspace of the stages' size; the smallest
        # workspace it accepts runs it in batches of queries, timed separately below)
        ws_full_b = (max(H.csa2_index_full_workspace(B, T, N, w.block, w.pool_blocks, K),
                         H.csa2_index_stages_workspace(B, T, N, w.block, w.pool_blocks, K)) if w.has_full else 0)
    ws_ri_b = H.csa2_reindex_workspace(max(w.n_reindex, 1), B, T, w.pool_cap, K)
    ws_attn_b = H.csa2_sparse_attn_workspace(L, B, T, Hh, K, w.swa_window)
    ws_full = torch.empty((max(ws_full_b, 1),), dtype=torch.uint8, device=dev)
    ws_attn = torch.empty((max(ws_attn_b, 1),), dtype=torch.uint8, device=dev)
    ws_ri = torch.empty((ws_ri_b,), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(512)
    ri_sets = sets[1:] if w.has_full else sets          # Reindex outputs follow the Full layer's set

    def scan(r):
        H.csa2_index_scan(k_rep[r], ks_rep[r], N, idx_q, head_w, n_vis, B, T, N, w.block, w.pool_blocks, K,
                          ws_full, ws_full_b)

    def full(r):
        H.csa2_index_full(k_rep[r], ks_rep[r], N, idx_q, head_w, n_vis, B, T, N, w.block, w.pool_blocks, K,
                          pool_pos, pool_len, sets[0], None, ws_full, ws_full_b)

    def select_reindex(r):
        n = w.n_reindex
        H.csa2_index_select_reindex(k_rep[r], ks_rep[r], N, n_vis, B, T, N, w.block, w.pool_blocks, K,
                                    ri_q if n else None, ri_w if n else None, n, pool_pos, pool_len,
                                    sets[0], None, ri_sets if n else None, None, ws_full, ws_full_b)

    def reindex(r):
        if w.n_reindex:
            H.csa2_reindex(k_rep[r], ks_rep[r], N, ri_q, ri_w, pool_pos, pool_len, w.pool_cap, w.n_reindex, B, T, K,
                           ri_sets, None, ws_ri, ws_ri_b)

    def attend(r):
        H.csa2_sparse_attn(codes_rep[r], scales_rep[r], N, qa, sets, list(w.layer_set), S, swa, w.swa_rows,
                           swa_end, w.swa_window, L, B, T, Hh, K, scale, out, lse, ws_attn, ws_attn_b)

    # The first stage is launched directly (and timed on its own); the others replay a graph.
    if chain:
        stages = (("scan", scan), ("pool, Full+Reindex top-k", select_reindex), ("attention", attend))
    elif w.has_full:
        stages = (("Full layer (scan, pool, top-k; batched)", full), ("reindex", reindex), ("attention", attend))
    else:
        stages = (("reindex", reindex), ("attention", attend))
    first = stages[0][1]

    def rest(r):
        for _, fn in stages[1:]:
            fn(r)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        if args.calibrate_copy:
            src_buf = torch.full((COPY_BYTES,), 1, dtype=torch.uint8, device=dev)
            dst_buf = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
            for _ in range(3):
                dst_buf.copy_(src_buf)
            torch.cuda.synchronize()
            del src_buf, dst_buf
        # eager warm-up and a per-stage breakdown (events on the launch stream, one stage at a time)
        for r in range(R):
            first(r)
            rest(r)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
        stage_ms = np.zeros(len(stages))
        reps = 10
        for i in range(reps):
            r = i % R
            ev[0].record()
            for j, (_, fn) in enumerate(stages):
                fn(r)
                ev[j + 1].record()
            ev[-1].synchronize()
            stage_ms += [ev[j].elapsed_time(ev[j + 1]) for j in range(len(stages))]
        stage_ms /= reps
        log("[bench] eager stage ms (serialised): " +
            "  ".join(f"{n} {v:.4f}" for (n, _), v in zip(stages, stage_ms)))
        min_ws_ms = None
        if w.has_full and not chain:
            # the Full layer in the smallest workspace csa2_index_full accepts (batches of queries)
            mws = H.csa2_index_full_workspace(B, T, N, w.block, w.pool_blocks, K)
            if mws < ws_full_b:
                ws_min = torch.empty((mws,), dtype=torch.uint8, device=dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                for i in range(reps + 2):
                    if i == 2:
                        e0.record()
                    H.csa2_index_full(k_rep[0], ks_rep[0], N, idx_q, head_w, n_vis, B, T, N, w.block,
                                      w.pool_blocks, K, pool_pos, pool_len, sets[0], None, ws_min, mws)
                e1.record()
                e1.synchronize()
                min_ws_ms = e0.elapsed_time(e1) / reps
                del ws_min
                log(f"[bench] Full layer in its smallest workspace ({mws / 2**20:.1f} MiB, batches of queries): "
                    f"{min_ws_ms:.4f} ms; with {ws_full_b / 2**20:.1f} MiB: {stage_ms[0]:.4f} ms")

        # Timed region: the first stage launched directly between timing events, the rest of
        # the step directly too (or from a HIP graph captured once per context replica).
        graphs = []
        if args.graph:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    rest(r)
                graphs.append(g)
        e_first = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]

        def run_step(i, timed=False):
            r = i % R
            if timed:
                e_first[i][0].record(stream)
            first(r)
            if timed:
                e_first[i][1].record(stream)
            if graphs:
                graphs[r].replay()
            else:
                rest(r)

        for i in range(args.warmup):
            run_step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run_step(i, timed=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall = t1 - t0
    first_ms = float(np.mean([a.elapsed_time(b) for a, b in e_first]))
    ms_per_step = wall * 1e3 / args.steps
    value = args.steps * Q / wall
    step_bytes = step_algorithmic_bytes(w)
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    copy_gbs = measure_copy_gbps(dev, stream) if not args.no_copy else None
    roofline = None
    if w.has_full:
        scan_bytes = scan_algorithmic_bytes(w)
        achieved = scan_bytes / (first_ms * 1e-3) / 1e9
        kernel_us = kernel_duration_from_profile("k_idx_scan", w.name)
        # without a pool the first stage is the whole batched Full layer, not the scan alone
        roofline = {"bound": "hbm", "kernel": "k_idx_scan" if chain else "csa2_index_full",
                    "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic_from_profile() if w.name == "decode_1m" else None,
                    "algorithmic_bytes_per_launch": scan_bytes, "avg_launch_us": round(first_ms * 1e3, 3),
                    # the event-bracketed launch above includes its dispatch; the committed rocprofv3
                    # kernel trace gives the kernel's own duration (None once the scan's sources change)
                    "frac_event": round(achieved / HBM_PEAK_GBS, 4),
                    "kernel_us_rocprof": kernel_us,
                    "frac_kernel": (round(scan_bytes / (kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                    if kernel_us else None),
                    # the whole step's algorithmic bytes over its wall time
                    "step_achieved": round(step_gbs, 1),
                    "step_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                    # the same figures against a plain device-to-device copy measured in this run
                    "copy_GBps": round(copy_gbs, 1) if copy_gbs else None,
                    "frac_of_copy": round(achieved / copy_gbs, 4) if copy_gbs else None,
                    "step_frac_of_copy": round(step_gbs / copy_gbs, 4) if copy_gbs else None}
        log(f"[bench] {args.steps} steps in {wall:.4f} s: {ms_per_step * 1e3:.2f} us/step, scan "
            f"{first_ms * 1e3:.2f} us ({achieved:.0f} GB/s algorithmic), whole step {step_gbs:.0f} GB/s algorithmic")
    else:
        log(f"[bench] {args.steps} steps in {wall:.4f} s: {ms_per_step * 1e3:.2f} us/step, reindex stage "
            f"{first_ms * 1e3:.2f} us, whole step {step_gbs:.0f} GB/s algorithmic")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "query_tokens": T, "context_entries": N,
                   "pool": f"{w.pool_blocks}x{w.block}" if w.pool_blocks else (
                       f"caller pools of {w.user_pool}" if w.user_pool else "none"),
                   "top_k": K, "full_layer": w.has_full, "reindex_layers": w.n_reindex,
                   "attention_layers": L, "attention_heads": Hh, "indexer_heads": 32, "indexer_dim": 128,
                   "indexer_keys": "fp4 (E2M1 + E4M3/16)" if w.idx_k_fp4 else "e4m3",
                   "indexer_query": "fp4 (E2M1 + E4M3/16)" if w.idx_k_fp4 else "e4m3",
                   "swa_window": w.swa_window, "context_replicas": R,
                   "launch": "first stage direct + hipgraph" if args.graph else "direct launches",
                   "step_algorithmic_bytes": step_bytes,
                   "step_algorithmic_GBps": round(step_gbs, 1),
                   "full_layer_workspace_bytes": ws_full_b if w.has_full else None,
                   "full_layer_min_workspace_ms": round(min_ws_ms, 4) if min_ws_ms else None},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
