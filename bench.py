#!/usr/bin/env python3
"""Benchmark of the HiLS-Attention forward hot path on one MI355X.

One step = one pass of the whole path over synthetic inputs already resident in
HBM: a 128K-token prefill forward (hils_summarize + hils_select +
hils_attend_fuse; B=1, 32 query / 8 KV heads, d=128, S=64, k=32, W=1024,
per-head scales U[0.5, 2]) followed by 256 decode steps over the 512K-token
caches of 4 sequences (hils_decode_step; k=32, W=1024; four chunk completions).
`value` is the prefill rate (tokens/s of the 128K forward); the decode rate is
reported beside it (decode_us_per_step, decode_us_per_token).  After the timed
steps, two more workloads are timed on their own: the 8K prefill (32/8 heads,
k=16, W=512) and 256 decode steps over one 4M-token cache (k=64, 8 needles).

Every call is timed with HIP events on the stream the library launches on
(torch's current stream); per-kernel durations come from the library's own
HIP-event timing.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HiLS fwd prefill tokens/s @128K + decode µs/token @512K; % HBM/MFMA roof"
PEAK_BF16 = 2.5e15      # dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12       # HBM3E, B/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def window_stats(T, S, W):
    i = np.arange(T, dtype=np.int64)
    a = i - W + 1
    lw = np.where(a > 0, (a // S) * S, 0)
    return lw // S, i - lw + 1       # |C_i|, |Win_i|


def num_cand(i, S, W):
    a = i - W + 1
    return 0 if a <= 0 else (a // S)


def attended_flops(B, Hq, T, d, S, W, k):
    nc, win = window_stats(T, S, W)
    return float(B * Hq * np.sum(4.0 * d * (np.minimum(k, nc) * S + win)))


def score_flops(B, Hq, T, d, S, W):
    nc, _ = window_stats(T, S, W)
    return float(B * Hq * np.sum(nc) * 2.0 * d)


def summary_bytes(B, Hq, Hkv, T, d, S, esz=2):
    NC = T // S
    return float(B * Hkv * NC * S * d * esz + 2 * B * Hq * NC * d * esz + B * Hq * NC * 4)


def decode_bytes(B, Hq, Hkv, d, S, W, k, positions, esz=2):
    """HBM bytes of decode steps at the given cache positions, B sequences each."""
    tot = 0.0
    for i in positions:
        a = i - W + 1
        lw = (a // S) * S if a > 0 else 0
        nc = lw // S
        win = i - lw + 1
        tot += Hq * nc * (d * esz + 4)                   # k', b' of every candidate
        tot += Hkv * min(k, nc) * S * d * esz * 2        # selected chunks' K and V
        tot += Hkv * win * d * esz * 2                   # window K and V
        tot += Hq * d * esz * 3 + Hkv * d * esz * 2      # q, q_hat, out; k_new, v_new
    return B * tot


def selected_entries(B, Hkv, T, S, W, k):
    nc, _ = window_stats(T, S, W)
    return float(B * Hkv * np.sum(np.minimum(k, nc)))


def attended_parts(B, Hq, T, d, S, W, k):
    """Attended FLOPs of the selected chunks and of the window (4d per attended
    (head, query, token): QK^T and PV), the two parts of sum_{i,h} 4d(min(k,|C_i|)S + |Win_i|)."""
    nc, win = window_stats(T, S, W)
    return (float(B * Hq * np.sum(4.0 * d * np.minimum(k, nc) * S)),
            float(B * Hq * np.sum(4.0 * d * win)))


def kernel_work(B, Hq, Hkv, T, d, S, W, k, esz=2):
    """Work of one launch of each prefill kernel: {kernel: (bound, amount, unit, design_bytes)}.

    The bound and amount are the ones the method prices the kernel on: attended
    FLOPs on the bf16 MFMA peak for the two attention kernels, score FLOPs for
    the score passes, HBM bytes for the memory-bound ones.  design_bytes counts
    each operand the kernel must move through HBM once in this design (no cache
    reuse assumed or credited); the counters' traffic is compared with it."""
    G = Hq // Hkv
    NC = T // S
    nc, win = window_stats(T, S, W)
    ncand = float(np.sum(nc))
    nsel = float(np.sum(np.minimum(k, nc)))
    ent = selected_entries(B, Hkv, T, S, W, k)
    rows = float(B * Hq * T)
    f_sel, f_win = attended_parts(B, Hq, T, d, S, W, k)
    sumb = summary_bytes(B, Hq, Hkv, T, d, S, esz)
    # per group: its rank keys and q_hat rows read once, its k' and b' once (the
    # chosen rows are gathered from L2), the index rows and each head's s_hat on
    # the choice written
    topk_b = B * Hkv * (ncand * 4.0 + T * G * d * esz + G * NC * (d * esz + 4.0) + T * k * 4.0
                        + G * nsel * 4.0)
    # K and V^T of every chunk once per KV head; per (query, group, slot) entry:
    # the entry word, G rows of q and G chunk weights read, G weighted partial
    # rows written
    chunk_b = float(B * Hkv * NC * S * d * esz * 2) + ent * (4 + G * d * esz * 2 + G * 4)
    # per row the q row, the selection normaliser, the row's partials, its
    # group's index row, the output and lse; K and V^T once per chunk and KV head
    win_b = (rows * (d * esz * 2 + 8) + B * Hq * nsel * d * esz + B * Hkv * T * k * 4.0
             + float(B * Hkv * NC * S * d * esz * 2))
    return {
        "summarize": ("hbm", sumb, "B", sumb),
        "score_lse": ("mfma", B * Hq * ncand * 2.0 * d, "FLOP", None),
        # these run once per pass of (b, KV group) pairs, every pair in one pass
        # with the full workspace: per launch, all B * Hkv groups' shares
        "rank_keys": ("mfma", B * Hkv * G * ncand * 2.0 * d, "FLOP", None),
        "topk_scores": ("hbm", topk_b, "B", topk_b),
        "chunk_attend": ("mfma", f_sel, "FLOP", chunk_b),
        "window": ("mfma", f_win, "FLOP", win_b),
    }


def overlap_m5(idx_t, T, S, W, k):
    """Mean fraction of a query's selected chunks that the next query also selected
    (rows where both have more candidates than k): the adjacent-query overlap
    that query packing would reuse."""
    import torch
    nc, _ = window_stats(T, S, W)
    x = idx_t.to(torch.int64)                                   # [B, Hkv, T, k]
    a, b = x[:, :, :-1, :], x[:, :, 1:, :]
    hit = (a.unsqueeze(-1) == b.unsqueeze(-2)).any(-1).sum(-1)  # [B, Hkv, T-1]
    rows = torch.from_numpy((nc[:-1] > k) & (nc[1:] > k)).to(x.device)
    n = int(rows.sum()) * x.shape[0] * x.shape[1]
    return float(hit[:, :, rows].sum()) / max(n * k, 1)


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# Sources a kernel's code depends on (its translation unit and every header it
# includes): a change to any voids its stored counters.
_CSRC = "chunk_wise_sparse_summary_amd/csrc/"
_HDRS = [_CSRC + h for h in ("hils_common.h", "hils_internal.h", "topk.h")]
_TILES = [_CSRC + "attend_tiles.h"]
KERNEL_SOURCES = {
    "summarize": [_CSRC + "summarize.hip"] + _HDRS,
    "score_lse": [_CSRC + "select.hip"] + _TILES + _HDRS,
    "rank_keys": [_CSRC + "select.hip"] + _TILES + _HDRS,
    "topk_scores": [_CSRC + "select.hip"] + _TILES + _HDRS,
    "window": [_CSRC + "attend.hip"] + _TILES + _HDRS,
    "chunk_attend": [_CSRC + "attend.hip"] + _TILES + _HDRS,
}


def stats_summary(csv_path, out_path, title, command):
    """Write a short text summary of a rocprofv3 --stats kernel table."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = ["# rocprofv3 kernel statistics: " + title,
             "# command (repository root, one MI355X):"] + ["#   " + c for c in command] + [
             "# source: %s; torch kernels generate the synthetic inputs." % csv_path, "",
             "%-64s %6s %14s %12s %8s" % ("kernel", "calls", "total_us", "avg_us", "pct")]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("void ", "").replace("hils::(anonymous namespace)::", "").replace("hils::", "")
        name = name.split("(")[0] if not name.startswith("__") else name
        t = float(r["TotalDurationNs"])
        lines.append("%-64s %6s %14.1f %12.1f %8.2f" % (name[:64], r["Calls"], t / 1e3,
                                                       t / 1e3 / max(int(r["Calls"]), 1), 100.0 * t / tot))
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_128k_prefill.txt")
COPY_PROBE_BYTES = 1 << 30


def read_traffic(kernel):
    """HBM bytes per launch of `kernel` from the stored counter summary, or None if
    absent or taken on a different version of the kernel's sources."""
    if not os.path.exists(TRAFFIC_FILE) or kernel not in KERNEL_SOURCES:
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            vals[key.strip()] = val.strip()
    if vals.get(kernel + ".source") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(vals[kernel + ".fetch_bytes"]) + float(vals[kernel + ".write_bytes"])
    except KeyError:
        return None


def ingest_pmc(fetch_csv, write_csv, command, out_path=TRAFFIC_FILE):
    """Turn two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE in KiB per dispatch)
    into per-launch HBM bytes of each library kernel, scaled by what the same
    counters read for the copy probe (a device copy of COPY_PROBE_BYTES)."""
    import csv

    def load(path, counter):
        # the last dispatch of each kernel is the one of the profiled prefill step
        per = {}
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v, did = r["Kernel_Name"], float(r["Counter_Value"]), int(r["Dispatch_Id"])
            if "copyBuffer" in name:
                copy.append(v)
            for kname in KERNEL_SOURCES:
                if "::%s_kernel" % kname in name and (kname not in per or did > per[kname][0]):
                    per[kname] = (did, v)
        return {kn: [v] for kn, (_, v) in per.items()}, max(copy) if copy else None

    fetch, cf = load(fetch_csv, "FETCH_SIZE")
    write, cw = load(write_csv, "WRITE_SIZE")
    if not cf or not cw:
        raise SystemExit("no copy-probe dispatch in the counter files")
    kib = COPY_PROBE_BYTES / 1024.0
    ff, fw = kib / cf, kib / cw
    lines = ["# HBM traffic per launch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE; KiB",
             "# per dispatch), scaled by the copy probe: a %d-byte device copy read"
             % COPY_PROBE_BYTES,
             "# FETCH_SIZE %.1f KiB and WRITE_SIZE %.1f KiB (factors %.4f, %.4f)." % (cf, cw, ff, fw),
             "# commands:"] + ["#   " + c for c in command] + [
             "copy_probe.fetch_factor = %.6f" % ff, "copy_probe.write_factor = %.6f" % fw]
    for kname in KERNEL_SOURCES:
        if not fetch.get(kname) or not write.get(kname):
            continue
        fb = float(np.mean(fetch[kname])) * 1024.0 * ff
        wb = float(np.mean(write[kname])) * 1024.0 * fw
        lines += ["%s.fetch_bytes = %.0f" % (kname, fb),
                  "%s.write_bytes = %.0f" % (kname, wb),
                  "%s.source = %s" % (kname, source_digest(KERNEL_SOURCES[kname]))]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def ingest_counters(csv_path, out_path, title, command):
    """Summarise a rocprofv3 counter run (any counters): for each library kernel, the
    mean per-dispatch value of each counter over its dispatches in the run."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"]
        if "hils::" not in name:
            continue
        kn = name.replace("void ", "").replace("hils::(anonymous namespace)::", "").replace("hils::", "")
        kn = kn.split("(")[0]
        per.setdefault(kn, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# rocprofv3 counters per dispatch (mean over the kernel's dispatches): " + title,
             "# command (repository root, one MI355X):"] + ["#   " + c for c in command] + [""]
    for kn in sorted(per):
        for cn in sorted(per[kn]):
            v = per[kn][cn]
            lines.append("%s.%s = %.6g    # %d dispatches" % (kn, cn, float(np.mean(v)), len(v)))
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_baseline(x, wl, seconds=10.0):
    """The fp64 oracle on the host: summaries of every chunk plus a sample of query
    rows, with all of the oracle's threads, then the same rows on one thread."""
    import oracle
    L = oracle.lib()
    threads = int(L.orc_max_threads())
    k_h = x["k"].cpu()
    ql_h = x["q_land"].cpu()
    t0 = time.perf_counter()
    ks, bs = oracle.summarize(k_h, ql_h, wl.S, wl.Hq, ks_round=oracle.ORND_BF16)
    t_sum = time.perf_counter() - t0
    v_h = x["v"].cpu()
    T = wl.T

    def rows_time(n):
        pos = np.linspace(T // 2, T - 1, n).astype(np.int64)
        q_rows = x["q"][:, :, pos].cpu()
        qh_rows = x["q_hat"][:, :, pos].cpu()
        rb, rg, rq = np.meshgrid(np.arange(wl.B), np.arange(wl.Hkv), np.arange(n), indexing="ij")
        rb, rg, rq = rb.ravel(), rg.ravel(), rq.ravel()
        t0_ = time.perf_counter()
        oracle.rows(rb, rg, pos[rq], rq, q_rows, qh_rows, k_h, v_h, ks, bs, S=wl.S, W=wl.W,
                    topk=wl.k)
        return time.perf_counter() - t0_

    n = 8
    while True:
        t_rows = rows_time(n)
        if t_rows + t_sum > seconds * 0.4 or n >= 512:
            break
        n *= 2
    per_token = t_sum / T + t_rows / n
    # one thread: the summaries of a 1/16 share of the chunks and 8 positions
    prev = oracle.set_threads(1)
    try:
        nc1 = (T // wl.S) // 16
        t0 = time.perf_counter()
        oracle.summarize(k_h, ql_h, wl.S, wl.Hq, ks_round=oracle.ORND_BF16, nc=nc1)
        t_sum1 = (time.perf_counter() - t0) * (T // wl.S) / nc1
        n1 = 8
        t_rows1 = rows_time(n1)
    finally:
        oracle.set_threads(prev)
    per_token1 = t_sum1 / T + t_rows1 / n1
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "single_core_value": 1.0 / per_token1,
            "sample": "128K prefill: fp64 summaries of all %d chunks x %d heads (%.1f s) plus all "
                      "%d KV groups of %d query positions from the second half of the sequence "
                      "(%.1f s) on %d threads; tokens/s = 1/(t_summaries/T + t_rows/positions). "
                      "single_core_value: one thread, summaries of %d chunks scaled to all "
                      "(%.1f s) plus %d positions (%.1f s)"
                      % (T // wl.S, wl.Hq, t_sum, wl.Hkv, n, t_rows, threads, nc1, t_sum1, n1,
                         t_rows1)}


def time_decode(hils, wl, cache, shape, ks, bs, steps, nrep, warm):
    """Per-step HIP-event times (ms) of `steps` decode steps from the cache length,
    run nrep times (positions restart each time; the cache rows they write and the
    summaries of the chunks they complete are rewritten with the same values)."""
    import torch
    dev = ks.device
    L0 = cache["length"]
    ws = hils.workspace(shape, hils.OP_DECODE, dev)
    dirs = cache["meta"].get("needle_dirs")
    import workloads as wk
    inputs = [wk.make_decode_step(wl, s, seed=cache["seed"], device=dev, needle_dirs=dirs)
              for s in range(steps)]
    out = torch.empty((wl.B, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.B, wl.Hkv, wl.k), dtype=torch.int32, device=dev)

    def one(s):
        st = inputs[s]
        hils.hils_decode_step([L0 + s] * wl.B, st["q"], st["q_hat"], st["k_new"], st["v_new"],
                              st["q_land_new"], cache["k_cache"], cache["v_cache"], ks, bs, out,
                              lse, idx, shape, ws)

    for s in range(warm):
        one(s)
    torch.cuda.synchronize()
    times = []
    for _ in range(nrep):
        ev = []
        for s in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record()
            one(s)
            b_.record()
            ev.append((a, b_))
        torch.cuda.synchronize()
        times += [a.elapsed_time(b_) for a, b_ in ev]
    return times


def time_decode_multi(hils, wl, cache, shape, ks, bs, M, calls, nrep=2, warm=4):
    """hils_decode_multi with M adjacent tokens per sequence: per-call HIP-event
    times (ms) of `calls` calls from the cache length (positions restart each
    repetition, as in time_decode), and per-kernel times of one more pass."""
    import torch
    import workloads as wk
    dev = ks.device
    L0 = cache["length"]
    nws = hils.hils_decode_multi_workspace_bytes(shape, M)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    inputs = []
    for c in range(calls):
        xs = [wk.make_decode_step(wl, c * M + m, seed=cache["seed"], device=dev) for m in range(M)]
        cat = lambda n: torch.stack([x[n] for x in xs], dim=1).contiguous()
        inputs.append({"q": cat("q"), "q_hat": cat("q_hat"), "k_new": cat("k_new"), "v_new": cat("v_new"),
                       "q_land_new": xs[-1]["q_land_new"]})
    out = torch.empty((wl.B, M, wl.Hq, wl.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((wl.B, M, wl.Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((wl.B, M, wl.Hkv, wl.k), dtype=torch.int32, device=dev)

    def one(c):
        st = inputs[c]
        hils.hils_decode_multi([L0 + c * M] * wl.B, M, st["q"], st["q_hat"], st["k_new"], st["v_new"],
                               st["q_land_new"], cache["k_cache"], cache["v_cache"], ks, bs, out, lse, idx,
                               shape, ws)
    for c in range(warm):
        one(c)
    torch.cuda.synchronize()
    times = []
    for _ in range(nrep):
        ev = []
        for c in range(calls):
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record()
            one(c)
            b_.record()
            ev.append((a, b_))
        torch.cuda.synchronize()
        times += [a.elapsed_time(b_) for a, b_ in ev]
    names = ["dec_append", "dec_score", "dec_select", "dec_gsel", "dec_attend", "dec_fuse", "dec_summarize"]
    hils.hils_timing_enable(names)
    for c in range(calls):
        one(c)
    torch.cuda.synchronize()
    kern = {}
    for kn in names:
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            kern[kn] = {"avg_us": tms / nl * 1e3, "launches_per_call": nl / calls}
    hils.hils_timing_enable(None)
    del ws
    return times, kern


PREFILL_KERNELS = ("summarize", "score_lse", "rank_keys", "topk_scores", "lsel", "idx_count",
                   "idx_scan_tiles", "idx_scan_buckets", "idx_fill", "v_transpose", "window",
                   "chunk_attend")
BWD_KERNELS = ["idx_count", "idx_scan_tiles", "idx_scan_buckets", "idx_fill", "bwd_rowstat", "bwd_kv",
               "bwd_dq", "bwd_qhat", "summarize_bwd"]


def time_backward(hils, x, fwd, shape, reps=3):
    """hils_attend_fuse_backward + hils_summarize_backward on the forward's own
    outputs (random upstream gradients), median of `reps` timed calls, then one
    call with per-kernel events."""
    import torch
    q = x["q"]
    dev = q.device
    B, Hq, T, d = q.shape
    Hkv = x["k"].shape[1]
    NC = T // shape.chunk
    gen = torch.Generator(device=dev)
    gen.manual_seed(77)
    dout = (torch.randn(q.shape, generator=gen, device=dev) * 0.5).to(q.dtype)
    dlse = torch.randn((B, Hq, T), generator=gen, device=dev) * 0.5
    f = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((B, Hq, T, d), **f), "dq_hat": torch.empty((B, Hq, T, d), **f),
         "dk": torch.empty((B, Hkv, T, d), **f), "dv": torch.empty((B, Hkv, T, d), **f),
         "dk_sum": torch.empty((B, Hq, NC, d), **f), "db_sum": torch.empty((B, Hq, NC), **f),
         "dq_land": torch.empty((B, Hq, NC, d), **f)}
    ws = hils.workspace(shape, hils.OP_ATTEND_BACKWARD, dev)

    def one():
        hils.hils_attend_fuse_backward(x["q"], x["k"], x["v"], x["q_hat"], fwd["k_sum"], fwd["idx"],
                                       fwd["ssel"], fwd["out"], fwd["lse"], dout, dlse, g["dq"], g["dk"],
                                       g["dv"], g["dq_hat"], g["dk_sum"], g["db_sum"], shape, ws)
        hils.hils_summarize_backward(x["k"], x["q_land"], g["dk_sum"], g["db_sum"], g["dk"], g["dq_land"],
                                     shape)
    one()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a.record()
        one()
        b_.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b_))
    hils.hils_timing_enable(BWD_KERNELS)
    one()
    torch.cuda.synchronize()
    kern = {}
    for kn in BWD_KERNELS:
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            kern[kn] = {"ms": tms, "launches": nl}
    hils.hils_timing_enable(None)
    ms = float(np.median(ts))
    af = attended_flops(B, Hq, T, d, shape.chunk, shape.window, shape.top_k)
    # five products per attended (row, token) pair instead of the forward's two:
    # S and U = dout V^T recomputed, then dV, dK and dq
    bf = 2.5 * af
    del ws, g
    return {"ms_median": ms, "attended_flops_bwd": bf,
            "mfma_frac": bf / (ms * 1e-3) / PEAK_BF16,
            "tokens_per_s": B * T / (ms * 1e-3),
            "kernels_ms": kern,
            "workspace_GiB": hils.hils_workspace_bytes(shape, hils.OP_ATTEND_BACKWARD) / 2**30,
            "note": "median of %d calls of attend_fuse_backward + summarize_backward; "
                    "FLOPs = 2.5 x the forward's attended FLOPs" % reps}


def time_bsa(hils, x, idx_hils, shape, ws, reps=2):
    """Naive-BSA selection (exact chunk masses, a diagnostic): median time of
    `reps` calls, and HiLS's recall against it over every row with a choice."""
    import torch
    q = x["q"]
    dev = q.device
    B, Hq, T, d = q.shape
    Hkv = x["k"].shape[1]
    S, W, k = shape.chunk, shape.window, shape.top_k
    bsa = torch.empty_like(idx_hils)

    def one():
        hils.hils_bsa_select(x["q"], x["k"], bsa, shape, ws)
    one()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a.record()
        one()
        b_.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b_))
    hils.hils_timing_enable(["bsa_keys", "bsa_topk"])
    one()
    torch.cuda.synchronize()
    kern = {}
    for kn in ("bsa_keys", "bsa_topk"):
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            kern[kn] = {"ms": tms, "launches": nl}
    hils.hils_timing_enable(None)
    cnt = torch.empty((B, Hkv, T), dtype=torch.int32, device=dev)
    hils.hils_selection_overlap(idx_hils, bsa, cnt, shape)
    torch.cuda.synchronize()
    i = np.arange(T)
    a_ = i - W + 1
    nc = np.where(a_ <= 0, 0, (a_ // S) * S) // S
    ev = nc > k
    hits = int(cnt.cpu().numpy()[:, :, ev].sum())
    n_ev = int(ev.sum()) * B * Hkv
    sweeps = 2 if Hq // Hkv > 1 else 1
    logits = float(B * Hq) * float(np.sum(nc)) * S     # (row, token) logits per sweep
    ms = float(np.median(ts))
    flops = sweeps * 2.0 * d * logits
    return {"ms_median": ms, "logit_flops": flops, "mfma_frac": flops / (ms * 1e-3) / PEAK_BF16,
            "exp_count": sweeps * logits, "kernels_ms": kern,
            "hils_recall": hits / (n_ev * k) if n_ev else None, "events": n_ev,
            "chance_recall": float(np.mean(k / nc[ev])) if ev.any() else None,
            "note": "exact chunk masses of every candidate (two sweeps for GQA) + wave top-k; "
                    "recall = shared chunk ids / (k x rows with |C_i| > k); chance = mean k/|C_i|"}


def time_qcal(hils, x, wl, shape, d_model=4096, rank=64, reps=5):
    """Q-Cal (q_hat = q + W_up W_down h) at the workload's size with random
    weights: median of `reps` calls; HBM roof on q, h and q_hat (the weights
    stay in cache).  Also the selection with Q-Cal fused into its scoring pass
    (hils_select_qcal) against Q-Cal followed by the selection."""
    import torch
    import workloads as wk
    q = x["q"]
    dev = q.device
    c = wk.make_qcal(wl, d_model, rank, seed=5, device=dev)
    qh = torch.empty_like(q)

    def med(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b_))
        return float(np.median(ts))

    ms = med(lambda: hils.hils_qcal(q, c["h"], c["w_down"], c["w_up"], qh, shape))
    esz = q.element_size()
    byts = 2 * q.numel() * esz + c["h"].numel() * esz + (c["w_down"].numel() + c["w_up"].numel()) * esz
    B, Hq, T, d = q.shape
    flops = 2.0 * B * T * rank * (d_model + Hq * d)
    res = {"ms_median": ms, "bytes": byts, "GBps": byts / (ms * 1e-3) / 1e9,
           "hbm_frac": byts / (ms * 1e-3) / PEAK_HBM, "flops": flops, "d_model": d_model, "rank": rank,
           "note": "median of %d calls; bytes = q + h + q_hat + weights" % reps}
    NC = T // wl.S
    ks = torch.empty((B, Hq, NC, d), dtype=q.dtype, device=dev)
    bs = torch.empty((B, Hq, NC), dtype=torch.float32, device=dev)
    hils.hils_summarize(x["k"], x["q_land"], ks, bs, shape)
    idx = torch.empty((B, wl.Hkv, T, wl.k), dtype=torch.int32, device=dev)
    sc = torch.empty((B, Hq, T, wl.k), dtype=torch.float32, device=dev)
    ws = torch.empty(hils.hils_select_qcal_workspace_bytes(shape, rank), dtype=torch.uint8, device=dev)
    # the selection's own workspace sits after z in the fused call's; same size here
    ws_sel = ws[ws.numel() - hils.hils_workspace_bytes(shape, hils.OP_SELECT):]
    sel_ms = med(lambda: hils.hils_select(qh, ks, bs, idx, sc, shape, ws_sel))
    fused_ms = med(lambda: hils.hils_select_qcal(q, c["h"], c["w_down"], c["w_up"], ks, bs, qh, idx, sc,
                                                 shape, ws))
    res["select_ms_median"] = sel_ms
    res["qcal_then_select_ms"] = ms + sel_ms
    res["select_qcal_fused_ms_median"] = fused_ms
    del c, qh, ks, bs, idx, sc, ws, ws_sel
    return res


def time_prefill_512k(hils, dev, reps=2):
    """The 512K context as one prefill (B=1, 32/8 heads, d=128, S=64, k=32, W=1024,
    per-head scales): 8192 chunks, selection and chunk pass one KV group at a time
    (workspaces of one group's share).  Median of `reps` calls after a warm-up,
    and a per-kernel breakdown from one more call."""
    import torch
    import workloads as wk
    wl = wk.custom(name="512k_prefill", kind="prefill", dtype="bf16", B=1, Hq=32, Hkv=8, d=128,
                   T=524288, S=64, k=32, W=1024, head_scale=(0.5, 2.0))
    x = wk.make_prefill(wl, seed=5, device=dev)
    sh = hils.Shape.make(wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T, torch.bfloat16)
    G = wl.Hq // wl.Hkv
    per_sel = wl.T * 64 * 128 * 4
    per_att = wl.T * wl.k * G * wl.d * 2
    wss = torch.empty(hils.hils_workspace_bytes(sh, hils.OP_SELECT) - (wl.B * wl.Hkv - 1) * per_sel,
                      dtype=torch.uint8, device=dev)
    wsa = torch.empty(hils.hils_workspace_bytes(sh, hils.OP_ATTEND_FUSE) - (wl.Hkv - 1) * per_att,
                      dtype=torch.uint8, device=dev)

    def run():
        return hils.prefill(x["q"], x["k"], x["v"], x["q_land"], x["q_hat"], S=wl.S, W=wl.W, topk=wl.k,
                            ws_select=wss, ws_attend=wsa)
    run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b_.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b_))
    ms = float(np.median(ts))
    names = list(PREFILL_KERNELS)
    hils.hils_timing_enable(names)
    run()
    torch.cuda.synchronize()
    kern = {}
    for kn in names:
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            kern[kn] = {"ms": tms, "launches": nl}
    hils.hils_timing_enable(None)
    af = attended_flops(wl.B, wl.Hq, wl.T, wl.d, wl.S, wl.W, wl.k)
    del x, wss, wsa
    return {"ms_median": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3), "attended_flops": af,
            "mfma_frac": af / (ms * 1e-3) / PEAK_BF16, "kernels_ms": kern,
            "note": "median of %d calls of summarize + select + attend_fuse after a warm-up; "
                    "one KV group per selection and chunk pass (16 + 22 GiB of workspace)" % reps}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=256,
                    help="decode steps per bench step (256: four chunk completions)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 8K prefill and 4M decode legs")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run a %d-byte device copy first (counter calibration)" % COPY_PROBE_BYTES)
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic summary from two rocprofv3 counter runs and exit")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("CSV", "OUT", "TITLE"),
                    help="write a per-kernel summary of a rocprofv3 counter run and exit")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="with --ingest-pmc / --ingest-counters / --stats-summary: the "
                         "profiling command lines, for the record")
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE,
                    help="with --ingest-pmc: where to write the summary")
    ap.add_argument("--stats-summary", nargs=3, metavar=("STATS_CSV", "OUT", "TITLE"),
                    help="write a text summary of a rocprofv3 --stats kernel table and exit")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.pmc_command, args.traffic_out)
        return
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters, args.pmc_command)
        return
    if args.stats_summary:
        stats_summary(args.stats_summary[0], args.stats_summary[1], args.stats_summary[2], args.pmc_command)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the HiLS path here runs on a single device and has "
              "no multi-GPU mode (--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import chunk_wise_sparse_summary_amd as hils
    import workloads as wk

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = wk.CONFIGS["128k"]
    dl = wk.CONFIGS["512k_decode"]
    log("generating 128K prefill inputs on device")
    x = wk.make_prefill(wl, seed=0, device=dev)
    B, Hq, Hkv, d, S, W, k, T = wl.B, wl.Hq, wl.Hkv, wl.d, wl.S, wl.W, wl.k, wl.T
    NC = T // S
    shape = hils.Shape.make(B, Hq, Hkv, d, S, W, k, T, torch.bfloat16)
    k_sum = torch.empty((B, Hq, NC, d), dtype=torch.bfloat16, device=dev)
    b_sum = torch.empty((B, Hq, NC), dtype=torch.float32, device=dev)
    idx = torch.empty((B, Hkv, T, k), dtype=torch.int32, device=dev)
    ssel = torch.empty((B, Hq, T, k), dtype=torch.float32, device=dev)
    out = torch.empty_like(x["q"])
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    ws_sel = hils.workspace(shape, hils.OP_SELECT, dev)
    ws_att = hils.workspace(shape, hils.OP_ATTEND_FUSE, dev)
    log("workspaces: select %.2f GiB, attend %.2f GiB" % (ws_sel.numel() / 2**30, ws_att.numel() / 2**30))

    log("generating 512K decode caches on device")
    cache = wk.make_decode_cache(dl, seed=1, device=dev)
    cache["seed"] = 1
    cap = cache["capacity"]
    dshape = hils.Shape.make(dl.B, dl.Hq, dl.Hkv, dl.d, dl.S, dl.W, dl.k, cap, torch.bfloat16)
    dks = torch.empty((dl.B, dl.Hq, cap // dl.S, dl.d), dtype=torch.bfloat16, device=dev)
    dbs = torch.empty((dl.B, dl.Hq, cap // dl.S), dtype=torch.float32, device=dev)
    ws_dec = hils.workspace(dshape, hils.OP_DECODE, dev)
    L0 = cache["length"]
    # summaries of the initial cache (also the summary-bandwidth measurement)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    sum_ms = []
    for rep in range(3):
        ev[0].record()
        hils.hils_summarize(cache["k_cache"], cache["q_land"], dks, dbs, dshape, 0, L0 // dl.S)
        ev[1].record()
        torch.cuda.synchronize()
        sum_ms.append(ev[0].elapsed_time(ev[1]))
    sum_dec_bytes = summary_bytes(dl.B, dl.Hq, dl.Hkv, L0, dl.d, dl.S)
    nsteps = min(args.decode_steps, cap - L0)
    dsteps = [wk.make_decode_step(dl, s, seed=1, device=dev) for s in range(nsteps)]
    dout = torch.empty((dl.B, dl.Hq, dl.d), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((dl.B, dl.Hq), dtype=torch.float32, device=dev)
    didx = torch.empty((dl.B, dl.Hkv, dl.k), dtype=torch.int32, device=dev)

    names = ["summarize", "select", "attend_fuse", "decode"]
    times = {n_: [] for n_ in names}

    def step():
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record()
        hils.hils_summarize(x["k"], x["q_land"], k_sum, b_sum, shape)
        e[1].record()
        hils.hils_select(x["q_hat"], k_sum, b_sum, idx, ssel, shape, ws_sel)
        e[2].record()
        hils.hils_attend_fuse(x["q"], x["k"], x["v"], idx, ssel, out, lse, shape, ws_att)
        e[3].record()
        de = []
        for s in range(nsteps):    # every step restarts at the same cache length
            st = dsteps[s]
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record()
            hils.hils_decode_step([L0 + s] * dl.B, st["q"], st["q_hat"], st["k_new"], st["v_new"],
                                  st["q_land_new"], cache["k_cache"], cache["v_cache"], dks, dbs,
                                  dout, dlse, didx, dshape, ws_dec)
            b_.record()
            de.append((a, b_))
        e[4].record()
        return e, de

    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # per-kernel HIP events around the prefill kernels only: events between the
    # few-microsecond decode kernels would stretch the decode step they measure
    timed_kernels = list(PREFILL_KERNELS)
    dec_kernels = ["dec_score", "dec_select", "dec_attend", "dec_fuse", "dec_summarize"]
    log("warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timed steps")
    recs = []
    hils.hils_timing_enable(timed_kernels)   # per-kernel HIP events on the launch stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(args.steps):
        recs.append(step())
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = g0.elapsed_time(g1)
    ktime = {}
    for kn in timed_kernels:
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            ktime[kn] = (tms / nl, nl / args.steps)   # ms per launch, launches per step
    hils.hils_timing_enable(None)
    for e, de in recs:
        times["summarize"].append(e[0].elapsed_time(e[1]))
        times["select"].append(e[1].elapsed_time(e[2]))
        times["attend_fuse"].append(e[2].elapsed_time(e[3]))
        for a, b_ in de:
            times["decode"].append(a.elapsed_time(b_))
    avg = {n_: float(np.mean(v)) if v else float("nan") for n_, v in times.items()}
    med = {n_: float(np.median(v)) if v else float("nan") for n_, v in times.items()}
    ms_per_step = total_ms / args.steps
    prefill_ms = avg["summarize"] + avg["select"] + avg["attend_fuse"]
    m5_128k = overlap_m5(idx, T, S, W, k)

    af = attended_flops(B, Hq, T, d, S, W, k)
    sf = score_flops(B, Hq, T, d, S, W)
    sb = summary_bytes(B, Hq, Hkv, T, d, S)
    dpositions = [L0 + s for s in range(nsteps)]
    db = decode_bytes(dl.B, dl.Hq, dl.Hkv, dl.d, dl.S, dl.W, dl.k, dpositions) / max(len(dpositions), 1)
    parts = {
        "summarize": {"bound": "hbm", "work": sb, "unit": "GB/s", "peak": PEAK_HBM},
        "select": {"bound": "mfma", "work": sf, "unit": "TFLOP/s", "peak": PEAK_BF16},
        "attend_fuse": {"bound": "mfma", "work": af, "unit": "TFLOP/s", "peak": PEAK_BF16},
        "prefill": {"bound": "mfma", "work": af, "unit": "TFLOP/s", "peak": PEAK_BF16},
        "decode": {"bound": "hbm", "work": db, "unit": "GB/s", "peak": PEAK_HBM},
    }
    avg["prefill"] = prefill_ms
    med["prefill"] = float(np.median([a_ + b_ + c_ for a_, b_, c_ in zip(times["summarize"], times["select"],
                                                                       times["attend_fuse"])]))
    kw = kernel_work(B, Hq, Hkv, T, d, S, W, k)
    kernels = {}
    for kn, (ms_l, per_step) in ktime.items():
        ent = {"avg_launch_ms": ms_l, "launches_per_step": per_step}
        if kn in kw:
            bound, amount, u, dbytes = kw[kn]
            rate = amount / (ms_l * 1e-3)
            ent.update({"bound": bound, "work_per_launch": amount,
                        "achieved": rate / (1e9 if u == "B" else 1e12),
                        "unit": "GB/s" if u == "B" else "TFLOP/s",
                        "frac": rate / (PEAK_HBM if u == "B" else PEAK_BF16)})
            if dbytes is not None:
                ent["design_bytes_per_launch"] = dbytes
                ent["design_GBps"] = dbytes / (ms_l * 1e-3) / 1e9
                tr = read_traffic(kn)
                if tr is not None:
                    ent["counter_bytes_per_launch"] = tr
        kernels[kn] = ent
    pre_k = [kn for kn in kernels if kn in kw]
    dom = max(pre_k, key=lambda kn: kernels[kn]["avg_launch_ms"] * kernels[kn]["launches_per_step"])
    kd = kernels[dom]
    roof = {"bound": kd["bound"], "kernel": dom + "_kernel", "achieved": kd["achieved"],
            "peak": (PEAK_HBM / 1e9) if kd["unit"] == "GB/s" else (PEAK_BF16 / 1e12),
            "unit": kd["unit"], "frac": kd["frac"], "traffic": read_traffic(dom),
            "work_per_launch": kd["work_per_launch"], "avg_launch_ms": kd["avg_launch_ms"]}
    if "design_bytes_per_launch" in kd:
        roof["bytes_roof"] = {"design_bytes": kd["design_bytes_per_launch"],
                              "achieved_GBps": kd["design_GBps"],
                              "frac": kd["design_GBps"] * 1e9 / PEAK_HBM,
                              "counter_bytes": roof["traffic"]}
    breakdown = {}
    for n_, pp in parts.items():
        a_ = pp["work"] / (avg[n_] * 1e-3)
        breakdown[n_] = {"avg_ms": avg[n_], "median_ms": med[n_], "bound": pp["bound"],
                         "achieved": a_ / (1e9 if pp["unit"] == "GB/s" else 1e12),
                         "unit": pp["unit"], "frac": a_ / pp["peak"]}
    res = {
        "metric": METRIC,
        "value": B * T / (prefill_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "128K prefill (B=1, 32q/8kv, d=128, S=64, k=32, W=1024) + %d decode "
                               "steps over 512K caches (B=4, k=32, W=1024)" % nsteps,
                   "value": "128K prefill tokens/s (summarize + select + attend_fuse)",
                   "prefill_tokens": B * T, "decode_batch": dl.B, "decode_cache_len": L0,
                   "decode_steps": nsteps},
        "prefill_ms": prefill_ms,
        "prefill_mfma_frac": breakdown["prefill"]["frac"],
        "decode_us_per_step": avg["decode"] * 1e3,
        "decode_us_per_step_median": med["decode"] * 1e3,
        "decode_us_per_token": avg["decode"] * 1e3 / dl.B,
        "decode_hbm_frac": breakdown["decode"]["frac"],
        "summary_512k_cache_GBps": sum_dec_bytes / (min(sum_ms) * 1e-3) / 1e9,
        "m5_overlap_128k": m5_128k,
        "roofline": roof,
        "breakdown": breakdown,
        "kernels": kernels,
        "wall_s_timed": wall,
    }
    # decode kernel breakdown: one more pass of the decode steps with per-kernel
    # events (these stretch the step; the step time above is measured without them)
    hils.hils_timing_enable(dec_kernels)
    for s in range(nsteps):
        st = dsteps[s]
        hils.hils_decode_step([L0 + s] * dl.B, st["q"], st["q_hat"], st["k_new"], st["v_new"],
                              st["q_land_new"], cache["k_cache"], cache["v_cache"], dks, dbs,
                              dout, dlse, didx, dshape, ws_dec)
    torch.cuda.synchronize()
    res["decode_kernels_us"] = {}
    for kn in dec_kernels:
        tms, nl = hils.hils_timing_get(kn)
        if nl:
            res["decode_kernels_us"][kn] = {"avg_us": tms / nl * 1e3, "launches_per_step": nl / nsteps}
    hils.hils_timing_enable(None)
    del ws_dec
    if not args.no_extra:
        log("512K multi-query decode (4 adjacent tokens per sequence)")
        Mq = 4
        calls = max(1, nsteps // Mq)
        tm_, km_ = time_decode_multi(hils, dl, cache, dshape, dks, dbs, Mq, calls)
        pos_m = [L0 + s for s in range(calls * Mq)]
        # bytes of one call: the k' stream once per sequence (shared by the M queries),
        # the selected and window chunks of each token as for one query
        db1 = decode_bytes(dl.B, dl.Hq, dl.Hkv, dl.d, dl.S, dl.W, dl.k, pos_m) / len(pos_m)
        kprime = dl.B * dl.Hq * (num_cand(L0 + calls * Mq // 2, dl.S, dl.W)) * (dl.d * 2 + 4)
        us_call = float(np.mean(tm_)) * 1e3
        res["decode_multi_512k"] = {
            "queries_per_sequence": Mq, "calls": calls, "us_per_call": us_call,
            "us_per_call_median": float(np.median(tm_)) * 1e3,
            "us_per_token": us_call / (dl.B * Mq),
            "single_query_us_per_token": avg["decode"] * 1e3 / dl.B,
            "bytes_per_call": Mq * db1 - (Mq - 1) * kprime,
            "hbm_frac": (Mq * db1 - (Mq - 1) * kprime) / (us_call * 1e-6) / PEAK_HBM,
            "kernels_us": km_,
            "note": "mean of 2 x %d calls (each: 4 tokens for each of the 4 sequences); bytes count the "
                    "k' stream once per sequence" % calls}
    if not args.no_extra:
        log("128K backward")
        del ws_att
        res["backward_128k"] = time_backward(hils, x, {"k_sum": k_sum, "idx": idx, "ssel": ssel, "out": out,
                                                       "lse": lse}, shape)
        log("128K Q-Cal")
        res["qcal_128k"] = time_qcal(hils, x, wl, shape)
        log("128K naive-BSA selection")
        res["bsa_128k"] = time_bsa(hils, x, idx, shape, ws_sel, reps=1)

    if not args.no_extra:
        # ---- 8K prefill (32/8 heads, d=128, k=16, W=512, one planted needle)
        log("8K prefill")
        w8 = wk.CONFIGS["8k"]
        x8 = {kk: (v.to(dev) if isinstance(v, torch.Tensor) else v)
              for kk, v in wk.make_prefill(w8, seed=0).items()}
        p8 = {}

        def run8():
            return hils.prefill(x8["q"], x8["k"], x8["v"], x8["q_land"], x8["q_hat"], S=w8.S,
                                W=w8.W, topk=w8.k, ws_select=p8.get("wss"), ws_attend=p8.get("wsa"))
        sh8 = hils.Shape.make(w8.B, w8.Hq, w8.Hkv, w8.d, w8.S, w8.W, w8.k, w8.T, torch.bfloat16)
        p8["wss"] = hils.workspace(sh8, hils.OP_SELECT, dev)
        p8["wsa"] = hils.workspace(sh8, hils.OP_ATTEND_FUSE, dev)
        for _ in range(3):
            r8 = run8()
        torch.cuda.synchronize()
        t8 = []
        for _ in range(20):
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record()
            r8 = run8()
            b_.record()
            torch.cuda.synchronize()
            t8.append(a.elapsed_time(b_))
        ms8 = float(np.median(t8))
        af8 = attended_flops(w8.B, w8.Hq, w8.T, w8.d, w8.S, w8.W, w8.k)
        res["prefill_8k"] = {"ms_median": ms8, "tokens_per_s": w8.B * w8.T / (ms8 * 1e-3),
                             "attended_flops": af8,
                             "mfma_frac": af8 / (ms8 * 1e-3) / PEAK_BF16,
                             "m5_overlap": overlap_m5(r8["idx"], w8.T, w8.S, w8.W, w8.k),
                             "note": "median of 20 calls of summarize + select + attend_fuse "
                                     "(output buffers allocated inside each call)"}
        log("8K backward")
        res["backward_8k"] = time_backward(hils, x8, r8, sh8, reps=10)
        log("8K naive-BSA selection")
        res["bsa_8k"] = time_bsa(hils, x8, r8["idx"], sh8, p8["wss"], reps=5)
        del x8, p8, r8
        # ---- 4M decode (B=1, k=64, 8 needles, 256 steps with 4 chunk completions)
        log("4M decode: drawing the cache")
        w4 = wk.CONFIGS["4m_decode"]
        c4 = wk.make_decode_cache(w4, seed=2, device=dev)
        c4["seed"] = 2
        cap4 = c4["capacity"]
        sh4 = hils.Shape.make(w4.B, w4.Hq, w4.Hkv, w4.d, w4.S, w4.W, w4.k, cap4, torch.bfloat16)
        ks4 = torch.empty((w4.B, w4.Hq, cap4 // w4.S, w4.d), dtype=torch.bfloat16, device=dev)
        bs4 = torch.empty((w4.B, w4.Hq, cap4 // w4.S), dtype=torch.float32, device=dev)
        s4 = []
        for _ in range(2):
            ev[0].record()
            hils.hils_summarize(c4["k_cache"], c4["q_land"], ks4, bs4, sh4, 0, c4["length"] // w4.S)
            ev[1].record()
            torch.cuda.synchronize()
            s4.append(ev[0].elapsed_time(ev[1]))
        log("4M decode: 256 steps")
        t4 = time_decode(hils, w4, c4, sh4, ks4, bs4, min(256, cap4 - c4["length"]), 2, 8)
        hils.hils_timing_enable(dec_kernels)
        time_decode(hils, w4, c4, sh4, ks4, bs4, min(256, cap4 - c4["length"]), 1, 0)
        k4 = {}
        for kn in dec_kernels:
            tms, nl = hils.hils_timing_get(kn)
            if nl:
                k4[kn] = {"avg_us": tms / nl * 1e3, "launches": nl}
        hils.hils_timing_enable(None)
        pos4 = [c4["length"] + s_ for s_ in range(min(256, cap4 - c4["length"]))]
        db4 = decode_bytes(w4.B, w4.Hq, w4.Hkv, w4.d, w4.S, w4.W, w4.k, pos4) / len(pos4)
        us4 = float(np.mean(t4)) * 1e3
        res["decode_4m"] = {"us_per_step": us4, "us_per_step_median": float(np.median(t4)) * 1e3,
                            "bytes_per_step": db4, "hbm_frac": db4 / (us4 * 1e-6) / PEAK_HBM,
                            "summary_GBps": summary_bytes(w4.B, w4.Hq, w4.Hkv, c4["length"], w4.d, w4.S)
                                            / (min(s4) * 1e-3) / 1e9,
                            "kernels_us": k4,
                            "note": "mean of 2 x 256 individually timed steps from 4194304 tokens "
                                    "(4 chunk completions per pass); kernels_us from a third pass "
                                    "with per-kernel events"}
        del c4, ks4, bs4
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        # ---- 512K prefill (the 512K context in one prefill: 8192 chunks)
        log("512K prefill")
        res["prefill_512k"] = time_prefill_512k(hils, dev)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(x, wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
