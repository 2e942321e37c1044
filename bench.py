#!/usr/bin/env python3
"""Throughput of the shifted-window attention hot path on one MI355X.

A step is one DiT block's attention on the FLUX-like 2048px image shape
(128x128 = 16384 tokens, 24 heads, head dim 128, bf16): the block's window
shift from the 4-phase schedule, mean pooling of K/V into 256 memory tokens
(8x8 cells), and shifted-window attention over [window keys; memory keys].
Steps cycle through the 4 schedule phases and through several input sets
(> 1 GB in total, so no step finds its inputs in the 256 MB last-level
cache); inputs are resident in HBM before timing starts.

Printed: one JSON line.  ``value`` is the window-attention algorithmic
TFLOP/s per step (4*B*H*n*(m+G)*D flops over the step time, pool included).
Both windows (16x16 and 32x32) are measured; ``--window`` picks the headline.
The dense kernel of the same library is timed at the same shape for the
realised-versus-theoretical speedup, and the CPU oracle is timed on a
bounded sample (``cpu_baseline``).
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (vendor figure)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (vendor figure)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "window_attn_traffic.json")
KERNEL_SOURCES = ["sparse_window_attention_amd/csrc/attn_bf16.hip",
                  "sparse_window_attention_amd/csrc/basa_internal.h",
                  "sparse_window_attention_amd/csrc/basa_common.h"]


# Workloads of --only profile: (workload name in workloads/, kernels run).
PROFILE_WORKLOADS = {
    "flux2048_w16": ("FLUX2048_W16", "window"),
    "flux2048_w32": ("FLUX2048_W32", "window"),
    "flux1024": ("FLUX1024", "window"),
    "wan": ("WAN", "window"),
    "wan_g1638": ("WAN_G1638", "window"),
    "ultra": ("ULTRA", "window"),
    "dense_flux2048": ("FLUX2048_W16", "dense"),
    "backward_flux2048_w16": ("FLUX2048_W16", "backward"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--window", type=int, default=16, choices=(16, 32))
    ap.add_argument("--sets", type=int, default=4, help="rotated input sets")
    ap.add_argument("--dense-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--only", choices=("window", "dense", "copy", "backward", "hilbert", "calib",
                                       "video", "pool", "profile", "all"),
                    default="all",
                    help="'window': only the headline steps; 'dense': only the dense kernel "
                         "at the same shape; 'copy': a plain device copy of known size, the "
                         "calibration for hardware byte counters (all three for profilers)")
    ap.add_argument("--shapes", default="flux1024,wan,wan_g1638,ultra,tiny_f32",
                    help="with --only video: comma-separated shapes to time")
    ap.add_argument("--workload", choices=tuple(PROFILE_WORKLOADS), default="flux2048_w16",
                    help="with --only profile: the workload whose kernels a few calls run "
                         "(for a counter profiler)")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="no GPU: read the rocprofv3 counter runs DIR/<workload>/<pass>/ and "
                         "DIR/copy/{fetch,write}/ and print one markdown table per workload")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="no GPU: read rocprofv3 outputs under DIR (ktrace/, pmc_fetch/, "
                         "pmc_write/, pmc_copy_fetch/, pmc_copy_write/), write the calibrated "
                         "HBM traffic of the attention kernel and print the summaries")
    return ap.parse_args()


# Work model of one call (algorithmic: the work the method must do, not the
# padding or L2 re-reads an implementation adds).
def window_flops(B, H, n, m, G, D):
    return 4 * B * H * n * (m + G) * D


def dense_flops(B, H, n, D):
    return 4 * B * H * n * n * D


def kernel_hash():
    """Hash of the attention kernel's code: line comments, indentation and
    blank lines are left out (the sources hold no block comments and no "//"
    in literals), so a change of comments alone keeps the counter summary."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def make_sets(wl, nsets, dev):
    import torch
    import workloads as W
    sets = []
    for s in range(nsets):
        q, k, v = W.make_qkv(wl, variant=s)
        sets.append(tuple(torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v)))
    return sets


def time_steps(S, wl, sets, steps, warmup, stream, with_mem=True):
    """Runs warmup + timed steps; returns (ms/step, pool ms list, attn ms list)."""
    import torch
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    G = wl.mem_tokens
    dev = sets[0][0].device
    outs = [torch.empty_like(s[0]) for s in sets]
    mems = [(torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev),
             torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev)) for _ in sets]

    def step(i, ev=None):
        si = i % len(sets)
        q, k, v = sets[si]
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        if ev is not None:
            ev[0].record(stream)
        mem = None
        if with_mem:
            mem = S.pool_kv(k, v, wl.grid, wl.pool, out=mems[si])
        if ev is not None:
            ev[1].record(stream)
        S.window_attn(q, k, v, wl.grid, wl.window, shift, mem=mem, out=outs[si])
        if ev is not None:
            ev[2].record(stream)

    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(warmup):
        step(i)
    host_s = (time.perf_counter() - h0) / max(warmup, 1)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # The host issues a step more slowly than the GPU runs it, so without a
    # backlog the queue runs dry and a host stall between an event and the
    # next launch would be counted as kernel time.  Queue GPU work lasting
    # about twice the host's issue time for all steps ahead of them; the
    # steps then run back to back from a full queue.
    backlog_ok = _queue_backlog(2.0 * steps * max(host_s, 1e-4) + 0.005, stream)
    t0.record(stream)
    for i in range(steps):
        step(warmup + i, evs[i])
    t1.record(stream)
    queued_ahead = backlog_ok and not t0.query()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    pool = [e[0].elapsed_time(e[1]) for e in evs]
    attn = [e[1].elapsed_time(e[2]) for e in evs]
    LAST_TIMING["queued_ahead"] = queued_ahead
    return total / steps, pool, attn


LAST_TIMING = {}
_BACKLOG = {}


def _queue_backlog(seconds, stream):
    """Enqueues plain bf16 matrix products lasting about `seconds` on the
    stream (their results are discarded).  The product's time is measured
    once.  Returns False if no product could be set up."""
    import torch
    try:
        if "mm" not in _BACKLOG:
            a = torch.randn((4096, 4096), device="cuda", dtype=torch.bfloat16)
            c = torch.empty_like(a)
            for _ in range(3):
                torch.mm(a, a, out=c)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                torch.mm(a, a, out=c)
            e1.record(stream)
            torch.cuda.synchronize()
            _BACKLOG["mm"] = (a, c, max(e0.elapsed_time(e1) / 10 * 1e-3, 1e-5))
        a, c, t_mm = _BACKLOG["mm"]
        for _ in range(min(int(math.ceil(seconds / t_mm)), 20000)):
            torch.mm(a, a, out=c)
        return True
    except RuntimeError:
        return False


def time_steps_graph(S, wl, sets, steps, warmup, stream, with_mem=True):
    """The same steps as time_steps, each replayed from a HIP graph captured
    per (input set, shift phase), with no events between the kernels: the
    whole-step time without host launches or per-kernel instrumentation.
    Each graph's output is checked bit for bit against an eager run of the
    same step (the kernels are deterministic).  Returns (ms/step, ok)."""
    import torch
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    G = wl.mem_tokens
    dev = sets[0][0].device
    outs = [torch.empty_like(s[0]) for s in sets]
    mems = [(torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev),
             torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev)) for _ in sets]
    period = len(sets) * 4 // math.gcd(len(sets), 4)

    def step(i, out=None):
        si = i % len(sets)
        q, k, v = sets[si]
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        mem = S.pool_kv(k, v, wl.grid, wl.pool, out=mems[si]) if with_mem else None
        S.window_attn(q, k, v, wl.grid, wl.window, shift, mem=mem,
                      out=outs[si] if out is None else out)

    for i in range(max(warmup, period)):
        step(i)
    torch.cuda.synchronize()
    graphs = []
    for i in range(period):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    # every graph against the eager step, with eager work and syncs between
    ok = True
    ref = torch.empty_like(outs[0])
    for i in range(period):
        graphs[i].replay()
        torch.cuda.synchronize()
        step(i, out=ref)
        torch.cuda.synchronize()
        ok = ok and torch.equal(outs[i % len(sets)], ref)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # the same start as the eager steps: behind a backlog, from a full queue
    backlog_ok = _queue_backlog(0.005 + steps * 2e-4, stream)
    t0.record(stream)
    for i in range(steps):
        graphs[i % period].replay()
    t1.record(stream)
    LAST_TIMING["graph_queued_ahead"] = backlog_ok and not t0.query()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, ok


def time_dense(S, sets, reps, stream):
    import torch
    q, k, v = sets[0]
    out = torch.empty_like(q)
    S.full_attn(q, k, v, out=out)
    torch.cuda.synchronize()
    ts = []
    for r in range(reps):
        q, k, v = sets[r % len(sets)]
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        S.full_attn(q, k, v, out=out)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return ts


def measure_mfma_peak(S, stream, reps=5):
    """bf16 MFMA rate of the library's calibration loop (no memory traffic),
    four workgroups of 8 waves per compute unit: the rate the matrix cores
    sustain on this chip at its clocks under full load."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 4 * cus, 4000
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    S.calib_mfma(sink, blocks, 200)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fl = S.calib_mfma(sink, blocks, iters)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = median(ts)
    return {"tflops": fl / (ms * 1e-3) / 1e12, "ms": ms, "flops": fl, "compute_units": cus,
            "note": "4 independent 32x32x16 bf16 MFMA chains per wave, 8 waves x 4 workgroups "
                    "per CU, register operands only"}


COPY_BYTES = 1 << 30   # bytes read (and again written) by one calibration copy


def time_copy(reps, stream):
    """A plain device-to-device copy of COPY_BYTES, the known-size reference that
    FETCH_SIZE / WRITE_SIZE are scaled by."""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return ts


def _counter_means(path, counter):
    """{kernel name: mean counter value per dispatch} from a rocprofv3 csv."""
    import csv
    import glob
    tot, disp = {}, {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = r["Kernel_Name"]
                tot[k] = tot.get(k, 0.0) + float(r["Counter_Value"])
                disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def _pick(d, key):
    hits = {k: v for k, v in d.items() if key in k}
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {list(hits)}")
    return next(iter(hits.items()))


def summarize_profiles(root):
    """Turns the byte-counter runs into calibrated HBM bytes per attention launch.

    FETCH_SIZE and WRITE_SIZE are read in KiB per dispatch; each is scaled by
    the ratio of the true bytes to what the same counter reads for the plain
    copy of COPY_BYTES."""
    import workloads as W
    wl = W.FLUX2048_W16
    copy_f = _pick(_counter_means(os.path.join(root, "pmc_copy_fetch"), "FETCH_SIZE"), "copy")[1]
    copy_w = _pick(_counter_means(os.path.join(root, "pmc_copy_write"), "WRITE_SIZE"), "copy")[1]
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    fetch = _counter_means(os.path.join(root, "pmc_fetch"), "FETCH_SIZE")
    write = _counter_means(os.path.join(root, "pmc_write"), "WRITE_SIZE")
    out = {"workload": wl.name, "kernel_source_hash": kernel_hash(),
           "copy_bytes": COPY_BYTES,
           "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    B, H, n, D, G = wl.batch, wl.heads, wl.n_tokens, wl.head_dim, wl.mem_tokens
    algo = {"attn_bf16": (3 * B * H * n * D * 2 + 2 * B * H * G * D * 2, B * H * n * D * 2),
            "pool_kernel": (2 * B * H * n * D * 2, 2 * B * H * G * D * 2)}
    for key, (ar, aw) in algo.items():
        name, fk = _pick(fetch, key)
        _, wk = _pick(write, key)
        rd, wr = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        out["kernels"][key] = {"name": name, "fetch_kib": fk, "write_kib": wk,
                               "read_bytes": rd, "write_bytes": wr,
                               "algorithmic_read_bytes": ar, "algorithmic_write_bytes": aw,
                               "read_over_algorithmic": rd / ar,
                               "write_over_algorithmic": wr / aw}
    a = out["kernels"]["attn_bf16"]
    out["hbm_bytes_per_launch"] = a["read_bytes"] + a["write_bytes"]
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    stats = os.path.join(root, "ktrace")
    import csv
    import glob
    for f in glob.glob(os.path.join(stats, "**", "*kernel_stats.csv"), recursive=True):
        print(f"\nkernel stats ({os.path.relpath(f, root)}):")
        with open(f) as fh:
            for r in csv.DictReader(fh):
                print(f"  {r['Name'][:90]:90s} calls {r['Calls']:>5s} avg_us "
                      f"{float(r['AverageNs']) / 1e3:9.2f} min_us {float(r['MinNs']) / 1e3:9.2f} "
                      f"max_us {float(r['MaxNs']) / 1e3:9.2f} pct {float(r['Percentage']):6.2f}")


COUNTER_PASSES = {
    "inst": "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_WAVES "
            "SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE",
    "busy": "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_LDS "
            "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE",
    "l2": "TCC_HIT_sum TCC_MISS_sum GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}


def _algorithmic(name, kernel):
    """(flops, read bytes, write bytes) the method needs for one dispatch of
    `kernel` in profile workload `name` (None where no clean split exists)."""
    import workloads as W
    wl = getattr(W, PROFILE_WORKLOADS[name][0])
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    m, G = wl.window_tokens, wl.mem_tokens
    t = B * H * n * D * 2
    if "pool_kernel" in kernel:
        return 0, 2 * t, 2 * B * H * G * D * 2
    import re
    full = re.search(r"attn_bf16\w*<\d+, (true|false)", kernel)
    if full and full.group(1) == "true":
        return dense_flops(B, H, n, D), 3 * t, t
    if full:
        return window_flops(B, H, n, m, G, D), 3 * t + 2 * B * H * G * D * 2, t
    return None


def summarize_counters(root):
    """Markdown tables of the counter runs under root (see COUNTER_PASSES and
    --only profile), one per workload: per kernel and dispatch, the MFMA
    products and their flops against the algorithmic flops, the share of
    cycles the matrix cores are busy, VALU instructions per MFMA, LDS bank
    conflicts, L2 hit rate, and HBM bytes (FETCH_SIZE / WRITE_SIZE scaled by
    what they read for a plain copy of COPY_BYTES) against the algorithmic
    bytes."""
    cf = _pick(_counter_means(os.path.join(root, "copy", "fetch"), "FETCH_SIZE"), "copy")[1]
    cw = _pick(_counter_means(os.path.join(root, "copy", "write"), "WRITE_SIZE"), "copy")[1]
    fs, ws = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    print(f"copy calibration: FETCH_SIZE x{fs:.3f}, WRITE_SIZE x{ws:.3f}\n")
    for name in PROFILE_WORKLOADS:
        d = os.path.join(root, name)
        if not os.path.isdir(d):
            continue
        c = {}
        for ps, ctrs in COUNTER_PASSES.items():
            for ctr in ctrs.split():
                for k, val in _counter_means(os.path.join(d, ps), ctr).items():
                    c.setdefault(k, {})[ctr] = val
        print(f"### {name}\n")
        print("| kernel | MFMA | MFMA GFLOP (algorithmic) | MFMA busy | VALU / MFMA | "
              "LDS conflicts / LDS inst | L2 hit | HBM read MB (algorithmic) | "
              "HBM write MB (algorithmic) |")
        print("|---|---|---|---|---|---|---|---|---|")
        for k in sorted(c):
            v = c[k]
            grbm = v.get("GRBM_GUI_ACTIVE", 0.0)
            mf = v.get("SQ_INSTS_MFMA", 0.0)
            busy = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024 * grbm / 8) if grbm else 0.0
            alg = _algorithmic(name, k)
            af = f" ({alg[0] / 1e9:.2f})" if alg and alg[0] else ""
            ar = f" ({alg[1] / 1e6:.1f})" if alg else ""
            aw = f" ({alg[2] / 1e6:.1f})" if alg else ""
            hits = v.get("TCC_HIT_sum", 0.0)
            miss = v.get("TCC_MISS_sum", 0.0)
            lds = v.get("SQ_ACTIVE_INST_LDS", 0.0)
            print(f"| {k[:60]} | {mf:.4g} | {mf * 32768 / 1e9:.2f}{af} | {busy:.1%} | "
                  f"{v.get('SQ_INSTS_VALU', 0.0) / mf if mf else 0.0:.2f} | "
                  f"{v.get('SQ_LDS_BANK_CONFLICT', 0.0) / lds if lds else 0.0:.3f} | "
                  f"{hits / (hits + miss) if hits + miss else 0.0:.1%} | "
                  f"{v.get('FETCH_SIZE', 0.0) * 1024 * fs / 1e6:.1f}{ar} | "
                  f"{v.get('WRITE_SIZE', 0.0) * 1024 * ws / 1e6:.1f}{aw} |")
        print()


def median(x):
    x = sorted(x)
    return x[len(x) // 2] if len(x) % 2 else 0.5 * (x[len(x) // 2 - 1] + x[len(x) // 2])


def pct(x, p):
    x = sorted(x)
    return x[min(len(x) - 1, max(0, int(round(p / 100.0 * (len(x) - 1)))))]


def cpu_baseline(wl, target_s):
    """The oracle, untuned, on a bounded sample of the headline workload:
    whole heads (every window, pooled memory) until ~target_s of CPU time."""
    import numpy as np
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    cache = {}
    calls, heads_done, flops, t_total = 0, 0, 0, 0.0
    # whole heads, cycling through the schedule phases, until ~target_s
    while t_total < target_s and heads_done < 32 * wl.heads:
        h, block = heads_done % wl.heads, heads_done // wl.heads
        if h not in cache:
            cache[h] = tuple(W.head_values(wl, t, h) for t in range(3))
        q, k, v = cache[h]
        shift = O.shift_for_block(block, wl.schedule, wl.window)
        t0 = time.perf_counter()
        km = O.pool_mean(k[None, None], wl.grid, wl.pool)[0, 0]
        vm = O.pool_mean(v[None, None], wl.grid, wl.pool)[0, 0]
        O.window_attention_head(q, k, v, wl.grid, wl.window, shift, km, vm)
        t_total += time.perf_counter() - t0
        heads_done += 1
        flops += O.window_flops(1, 1, wl.n_tokens, wl.window_tokens, wl.mem_tokens, wl.head_dim)
    tflops = flops / t_total / 1e12
    ms_per_call = t_total / heads_done * wl.heads * 1e3
    return {"value": tflops, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads_done} head-blocks (head x schedule phase, {wl.heads} heads per "
                      f"call) of {wl.name}, all {wl.n_windows} windows each, pool included, "
                      f"fp64 numpy; {t_total:.1f} s of oracle time",
            "ms_per_call_extrapolated": ms_per_call,
            "cpu": platform.processor() or platform.machine(), "os_cpu_count": os.cpu_count()}


def oracle_per_config():
    """The oracle beside the other shapes: one head of FLUX-1024, Wan and
    Ultra timed (block 1 of the schedule, pool included), the call's time
    extrapolated to all heads; Tiny by the brute-force masked definition."""
    import oracle as O
    import workloads as W
    res = {}
    for wl in (W.FLUX1024, W.WAN, W.ULTRA):
        q, k, v = (W.head_values(wl, t, 0) for t in range(3))
        shift = O.shift_for_block(1, wl.schedule, wl.window)
        t0 = time.perf_counter()
        km = O.pool_mean(k[None, None], wl.grid, wl.pool)[0, 0]
        vm = O.pool_mean(v[None, None], wl.grid, wl.pool)[0, 0]
        O.window_attention_head(q, k, v, wl.grid, wl.window, shift, km, vm)
        dt = time.perf_counter() - t0
        fl = O.window_flops(1, 1, wl.n_tokens, wl.window_tokens, wl.mem_tokens, wl.head_dim)
        res[wl.name] = {"ms_one_head": dt * 1e3,
                        "ms_per_call_extrapolated": dt * 1e3 * wl.heads * wl.batch,
                        "tflops": fl / dt / 1e12,
                        "note": f"one of {wl.heads} heads timed; the call extrapolated"}
        del q, k, v, km, vm
    wl = W.TINY
    q, k, v = W.make_qkv(wl)
    shift = (4, 4)
    t0 = time.perf_counter()
    O.masked_attention_bruteforce(q, k, v, wl.grid, wl.window, shift)
    res[wl.name] = {"ms_per_call": (time.perf_counter() - t0) * 1e3,
                    "note": "brute-force masked attention, the whole call (one head)"}
    return res


def window_permutation(grid, window, shift, device):
    """Raster index of every token in window-major order under the shifted
    partition: windows in raster order of the window grid, tokens in raster
    order inside each window, for the grid rolled by -shift.  One
    ``index_select`` with it materialises the roll and the partition (the
    copies a stock-backend deployment makes); its inverse undoes both."""
    import torch
    g, w, s = list(grid), list(window), list(shift)
    if len(g) == 2:
        g, w, s = [1] + g, [1] + w, [0] + s
    idx = torch.arange(g[0] * g[1] * g[2], dtype=torch.int64).view(*g)
    idx = torch.roll(idx, shifts=[-x for x in s], dims=(0, 1, 2))
    idx = idx.view(g[0] // w[0], w[0], g[1] // w[1], w[1], g[2] // w[2], w[2])
    perm = idx.permute(0, 2, 4, 1, 3, 5).reshape(-1)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(perm.numel(), dtype=torch.int64)
    return perm.to(device), inv.to(device)


def composition_index(B, H, grid, window, shift, device):
    """Row indices of the stock-backend composition over a [B*H*n, D] view
    of a BHND tensor: ``fwd`` takes it to window-batched order [B*nW, H, m,
    D] (the grid rolled by -shift and cut into windows: row (b, j, h, r) is
    token perm[j*m + r] of head (b, h)); ``inv`` takes a tensor in that
    order back to [B, H, n, D] raster order (unpartition and roll by +shift)."""
    import torch
    perm, _ = window_permutation(grid, window, shift, "cpu")
    n = perm.numel()
    m = int(math.prod(window))
    nW = n // m
    b = torch.arange(B).view(B, 1, 1, 1)
    j = torch.arange(nW).view(1, nW, 1, 1)
    h = torch.arange(H).view(1, 1, H, 1)
    r = torch.arange(m).view(1, 1, 1, m)
    fwd = ((b * H + h) * n + perm.view(nW, m)[j, r]).reshape(-1)
    inv = torch.empty_like(fwd)
    inv[fwd] = torch.arange(fwd.numel())
    return fwd.to(device), inv.to(device)


def compose_attention(S, q, k, v, mem, grid, window, shift, index=None, parts=None):
    """The composition a stock backend runs (BASA forum summary, "Overview": no custom
    operator, only existing dense attention kernels): materialised roll +
    window partition of Q, K and V (one gather each, into [B*nW, H, m, D]);
    each window's keys and values concatenated with the pooled memory (a
    broadcast copy, [B*nW, H, m+G, D]); one unmodified dense attention call
    over the B*nW window batches; then unpartition + unroll of O (a
    gather).  ``parts``, if given, is a list that receives HIP events
    bracketing the four phases."""
    import torch
    B, H, n, D = q.shape
    m = int(math.prod(window))
    nW = n // m
    fwd, inv = index or composition_index(B, H, grid, window, shift, q.device)
    ev = None
    if parts is not None:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record()
    qw, kw, vw = (x.view(-1, D).index_select(0, fwd).view(B * nW, H, m, D) for x in (q, k, v))
    if ev:
        ev[1].record()
    if mem is not None:
        G = mem[0].shape[2]
        kw, vw = (torch.cat([w.view(B, nW, H, m, D), x.unsqueeze(1).expand(B, nW, H, G, D)],
                            dim=3).view(B * nW, H, m + G, D)
                  for w, x in ((kw, mem[0]), (vw, mem[1])))
    if ev:
        ev[2].record()
    ow = S.dense_attn(qw, kw, vw)
    if ev:
        ev[3].record()
    out = ow.view(-1, D).index_select(0, inv).view(B, H, n, D)
    if ev:
        ev[4].record()
        parts.append(ev)
    return out


def measure_composition(S, wl, sets, steps, stream):
    """Times the composition baseline (events per phase) on the rotated input
    sets, beside the fused kernel it stands against."""
    import torch
    B, H = wl.batch, wl.heads
    shifts = [S.shift_for_block(i, wl.schedule, wl.window) for i in range(4)]
    dev = sets[0][0].device
    idx = [composition_index(B, H, wl.grid, wl.window, sh, dev) for sh in shifts]
    mems = [S.pool_kv(k, v, wl.grid, wl.pool) for (q, k, v) in sets]
    evs = []
    for i in range(steps + 2):
        q, k, v = sets[i % len(sets)]
        sink = [] if i >= 2 else None
        compose_attention(S, q, k, v, mems[i % len(sets)], wl.grid, wl.window, shifts[i % 4],
                          index=idx[i % 4], parts=sink)
        torch.cuda.synchronize()
        if sink:
            evs.append(sink[0])
    names = ("roll_partition_gather", "memory_concat", "dense_attention", "unpartition_unroll")
    r = {key: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / len(evs)
         for j, key in enumerate(names)}
    r["total"] = sum(r[key] for key in names)
    m, G, D, n = wl.window_tokens, wl.mem_tokens, wl.head_dim, wl.n_tokens
    tok = B * H * n * D * 2              # bytes of one bf16 [B, H, n, D] tensor
    kvc = B * (n // m) * H * (m + G) * D * 2   # one [B*nW, H, m+G, D] key or value tensor
    memb = B * H * G * D * 2
    r["bytes_moved"] = {
        "roll_partition_gather": 6 * tok,            # read and write Q, K, V
        "memory_concat": 2 * (tok + memb + kvc),     # read K/V windows and memory, write K/V+mem
        "dense_attention": 2 * tok + 2 * kvc,        # read Q, K, V, write O
        "unpartition_unroll": 2 * tok,               # read and write O
    }
    r["bytes_moved_total"] = sum(r["bytes_moved"].values())
    r["note"] = ("stock-backend composition: materialised roll+partition (one gather per "
                 "tensor into [B*nW, H, m, D]), memory concatenated to every window's K/V "
                 "([B*nW, H, m+G, D]), the library's dense kernel (basa_dense_attn) over the "
                 "window batches, then unpartition+unroll (a gather); HIP events per phase")
    return r


def measure_backward(S, wl, sets, steps, stream):
    """Times the training-side pair at the headline shape: the forward that
    also writes the log-sum-exp, then the backward (gradients of Q, K, V with
    the pooled memory's gradient folded back).  Algorithmic backward work:
    five products per window (S, dP, dV, dK, dQ), 10*B*H*n*(m+G)*D flops."""
    import torch
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    m, G = wl.window_tokens, wl.mem_tokens
    dev = sets[0][0].device
    douts = [torch.randn_like(s[0]) for s in sets]
    lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    outs = [torch.empty_like(s[0]) for s in sets]
    grads = tuple(torch.empty_like(sets[0][0]) for _ in range(3))
    ws = torch.empty(S.bwd_workspace_bytes(B, H, D, wl.grid, wl.pool), dtype=torch.uint8,
                     device=dev)
    fwd, bwd = [], []
    for i in range(steps + 3):
        q, k, v = sets[i % len(sets)]
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        mem = S.pool_kv(k, v, wl.grid, wl.pool)
        ev[0].record(stream)
        out, _ = S.window_attn_fwd(q, k, v, wl.grid, wl.window, shift, mem=mem,
                                   out=outs[i % len(sets)], lse=lse)
        ev[1].record(stream)
        S.window_attn_bwd(q, k, v, out, douts[i % len(sets)], lse, wl.grid, wl.window, shift,
                          mem=mem, pool=wl.pool, grads=grads, workspace=ws)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            fwd.append(ev[0].elapsed_time(ev[1]))
            bwd.append(ev[1].elapsed_time(ev[2]))
    fl = 10 * B * H * n * (m + G) * D
    f_ms, b_ms = sum(fwd) / len(fwd), sum(bwd) / len(bwd)
    return {"workload": wl.name, "forward_with_lse_ms": f_ms, "backward_ms": b_ms,
            "backward_algorithmic_flops": fl,
            "backward_tflops": fl / (b_ms * 1e-3) / 1e12,
            "backward_mfma_frac": fl / (b_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "workspace_bytes": ws.numel(),
            "note": "backward = dvec, memory-key dV/dK partials, their sum, window-key dV/dK "
                    "(pooled memory gradient folded in), dQ"}


def measure_other_shape(S, wl, stream, dev, steps, dense_reps):
    """Window attention (pool included, the workload's shift schedule) and the
    in-build dense kernel at another of the pages' shapes.  Inputs are N(0,1)
    drawn on the GPU (timing only; the seeded workload values are the parity
    tests' business)."""
    import torch
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    m, G = wl.window_tokens, wl.mem_tokens
    g = torch.Generator(device=dev)
    g.manual_seed(5000 + wl.seed)
    q, k, v = (torch.randn((B, H, n, D), generator=g, device=dev).to(torch.bfloat16)
               for _ in range(3))
    out = torch.empty_like(q)
    mem = tuple(torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev) for _ in range(2))
    pool, attn = [], []
    for i in range(steps + 3):
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        _queue_backlog(0.002, stream)   # the step's launches are issued before it runs
        ev[0].record(stream)
        S.pool_kv(k, v, wl.grid, wl.pool, out=mem)
        ev[1].record(stream)
        S.window_attn(q, k, v, wl.grid, wl.window, shift, mem=mem, out=out)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            pool.append(ev[0].elapsed_time(ev[1]))
            attn.append(ev[1].elapsed_time(ev[2]))
    a0 = []
    for i in range(max(3, steps // 2) + 2):
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        _queue_backlog(0.002, stream)
        ev[0].record(stream)
        S.window_attn(q, k, v, wl.grid, wl.window, shift, out=out)
        ev[1].record(stream)
        torch.cuda.synchronize()
        if i >= 2:
            a0.append(ev[0].elapsed_time(ev[1]))
    dense_ms = median(time_dense(S, [(q, k, v)], dense_reps, stream))
    p_ms, a_ms, a0_ms = (sum(x) / len(x) for x in (pool, attn, a0))
    fl = window_flops(B, H, n, m, G, D)
    r = {"workload": wl.name, "n": n, "m": m, "G": G, "pool_kv_ms": p_ms, "window_attn_ms": a_ms,
         "window_attn_tflops": fl / (a_ms * 1e-3) / 1e12,
         "window_attn_mfma_frac": fl / (a_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
         "window_attn_nomem_ms": a0_ms, "dense_ms": dense_ms,
         "dense_tflops": dense_flops(B, H, n, D) / (dense_ms * 1e-3) / 1e12,
         "speedup": {"theoretical_n_over_m": n / m, "realised_nomem": dense_ms / a0_ms,
                     "realised_over_theoretical_nomem": dense_ms / a0_ms / (n / m),
                     "theoretical_n_over_m_plus_G": n / (m + G), "realised_mem": dense_ms / a_ms,
                     "realised_over_theoretical_mem": dense_ms / a_ms / (n / (m + G)),
                     "realised_mem_incl_pool": dense_ms / (a_ms + p_ms)},
         "data": "synthetic N(0,1) on the GPU"}
    del q, k, v, out, mem
    torch.cuda.empty_cache()
    return r


def run_profile_workload(S, name, stream, dev, calls=3):
    """A few calls of one workload's kernels on N(0,1) inputs drawn on the
    GPU, for a counter profiler (every dispatch is averaged)."""
    import torch
    import workloads as W
    wl = getattr(W, PROFILE_WORKLOADS[name][0])
    kind = PROFILE_WORKLOADS[name][1]
    B, H, n, D = wl.batch, wl.heads, wl.n_tokens, wl.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(7000)
    q, k, v = (torch.randn((B, H, n, D), generator=g, device=dev).to(torch.bfloat16)
               for _ in range(3))
    out = torch.empty_like(q)
    for i in range(calls):
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        if kind == "dense":
            S.full_attn(q, k, v, out=out)
        elif kind == "window":
            mem = S.pool_kv(k, v, wl.grid, wl.pool)
            S.window_attn(q, k, v, wl.grid, wl.window, shift, mem=mem, out=out)
        else:
            mem = S.pool_kv(k, v, wl.grid, wl.pool)
            o, lse = S.window_attn_fwd(q, k, v, wl.grid, wl.window, shift, mem=mem, out=out)
            S.window_attn_bwd(q, k, v, o, q, lse, wl.grid, wl.window, shift, mem=mem,
                              pool=wl.pool)
        torch.cuda.synchronize()
    return {"workload": name, "calls": calls}


def measure_pool(S, stream, dev, steps):
    """The pool at FLUX-2048 (24 heads, 8x8 cells) two ways: alone (the GPU
    idle before each call) and in the step (right after a window attention
    launch, whose 100 MB of output is still being written)."""
    import torch
    import workloads as W
    wl = W.FLUX2048_W16
    B, H, n, D, G = wl.batch, wl.heads, wl.n_tokens, wl.head_dim, wl.mem_tokens
    sets = make_sets(wl, 5, dev)
    mem = tuple(torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev) for _ in range(2))
    out = torch.empty_like(sets[0][0])
    alone, instep = [], []
    c = 0   # each call takes the next of the 5 input sets: no call finds its
            # inputs in the last-level cache from the call before
    for i in range(steps + 2):
        shift = S.shift_for_block(i % 4, wl.schedule, wl.window)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        _queue_backlog(0.001, stream)
        ev[0].record(stream)
        q, k, v = sets[c % len(sets)]
        S.pool_kv(k, v, wl.grid, wl.pool, out=mem)
        ev[1].record(stream)
        torch.cuda.synchronize()
        _queue_backlog(0.001, stream)
        q, k, v = sets[(c + 1) % len(sets)]
        S.window_attn(q, k, v, wl.grid, wl.window, shift, mem=mem, out=out)
        ev[2].record(stream)
        q, k, v = sets[(c + 2) % len(sets)]
        S.pool_kv(k, v, wl.grid, wl.pool, out=mem)
        ev[3].record(stream)
        c += 3
        torch.cuda.synchronize()
        if i >= 2:
            alone.append(ev[0].elapsed_time(ev[1]))
            instep.append(ev[2].elapsed_time(ev[3]))
    byts = 2 * B * H * n * D * 2 + 2 * B * H * G * D * 2
    a, b = median(alone), median(instep)
    return {"workload": wl.name, "pool_alone_ms": a, "pool_in_step_ms": b,
            "algorithmic_bytes": byts, "alone_gbs": byts / (a * 1e-3) / 1e9,
            "in_step_gbs": byts / (b * 1e-3) / 1e9,
            "note": "alone: after the GPU idled (synchronised), behind a short backlog; in "
                    "step: launched right after a window attention call; every call on an "
                    "input set not touched by the two calls before it"}


def measure_tiny(S, stream, dev, steps):
    """The fp32 Tiny workload (16x16 tokens, one head, D = 64, 8x8 windows
    shifted by (4,4), no memory) through the fp32 kernels, and the fp32 dense
    kernel at the same shape; each call queued behind a short backlog."""
    import torch
    import workloads as W
    wl = W.TINY
    q, k, v = (torch.from_numpy(x).to(dev) for x in W.make_qkv(wl))
    out = torch.empty_like(q)
    win, dense = [], []
    for i in range(steps + 3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        _queue_backlog(0.001, stream)
        ev[0].record(stream)
        S.window_attn(q, k, v, wl.grid, wl.window, (4, 4), scale=1.0 / math.sqrt(64), out=out)
        ev[1].record(stream)
        S.full_attn(q, k, v, out=out)
        ev[2].record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            win.append(ev[0].elapsed_time(ev[1]))
            dense.append(ev[1].elapsed_time(ev[2]))
    n, m, D = wl.n_tokens, wl.window_tokens, wl.head_dim
    w_ms, d_ms = median(win), median(dense)
    return {"workload": wl.name, "dtype": "f32", "n": n, "m": m, "G": 0,
            "window_attn_ms": w_ms,
            "window_attn_gflops": window_flops(1, 1, n, m, 0, D) / (w_ms * 1e-3) / 1e9,
            "dense_ms": d_ms, "realised_over_theoretical": d_ms / w_ms / (n / m),
            "note": "fp32 vector-ALU kernels (an accuracy path, not a throughput one): one "
                    "workgroup per 128 queries, so a call is launch- and latency-bound"}


HILBERT_SIDES = (64, 128)    # token grids of 1024 x 1024 and 2048 x 2048 px images
HILBERT_TILE = 256
HILBERT_REGION = (8, 8)


def measure_hilbert(S, stream, dev, steps):
    """Attention in tiles of 256 consecutive Hilbert-curve positions, sliding
    half a tile from call to call, with an 8 x 8 central region as memory,
    against the in-build dense kernel at the same shape (B=1, 24 heads,
    D=128).  A step is the region gather plus the tile attention."""
    import torch
    res = {}
    for side in HILBERT_SIDES:
        n, B, H, D = side * side, 1, 24, 128
        g = torch.Generator(device=dev)
        g.manual_seed(4000 + side)
        sets = [tuple(torch.randn((B, H, n, D), generator=g, device=dev).to(torch.bfloat16)
                      for _ in range(3)) for _ in range(2)]
        order = torch.from_numpy(S.hilbert_order(side)).to(dev)
        reg = torch.from_numpy(S.center_region_tokens((side, side), HILBERT_REGION)).to(dev)
        G = reg.numel()
        out = torch.empty_like(sets[0][0])
        mem = tuple(torch.empty((B, H, G, D), dtype=torch.bfloat16, device=dev) for _ in range(2))
        gat, att, att0 = [], [], []
        for i in range(steps + 3):
            q, k, v = sets[i % 2]
            slide = (i % 2) * HILBERT_TILE // 2
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            _queue_backlog(0.002, stream)   # the step's launches are issued before it runs
            ev[0].record(stream)
            S.gather_kv(k, v, reg, out=mem)
            ev[1].record(stream)
            S.curve_attn(q, k, v, order, HILBERT_TILE, slide, mem=mem, out=out)
            ev[2].record(stream)
            S.curve_attn(q, k, v, order, HILBERT_TILE, slide, out=out)
            ev[3].record(stream)
            torch.cuda.synchronize()
            if i >= 3:
                gat.append(ev[0].elapsed_time(ev[1]))
                att.append(ev[1].elapsed_time(ev[2]))
                att0.append(ev[2].elapsed_time(ev[3]))
        # the gather is a few microseconds: events around one launch mostly time
        # the events, so it is also timed as a burst of launches back to back
        burst = 20
        _queue_backlog(0.002, stream)
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        eb[0].record(stream)
        for j in range(burst):
            S.gather_kv(sets[j % 2][1], sets[j % 2][2], reg, out=mem)
        eb[1].record(stream)
        torch.cuda.synchronize()
        g_burst = eb[0].elapsed_time(eb[1]) / burst
        dense_ms = median(time_dense(S, sets, 3, stream))
        g_ms, a_ms, a0_ms = (sum(x) / len(x) for x in (gat, att, att0))
        fl = window_flops(B, H, n, HILBERT_TILE, G, D)
        res[f"{side}x{side}"] = {
            "n": n, "tile": HILBERT_TILE, "region_tokens": G,
            "gather_ms": g_burst, "gather_ms_one_launch_events": g_ms,
            "tile_attn_ms": a_ms, "tile_attn_nomem_ms": a0_ms,
            "tile_attn_tflops": fl / (a_ms * 1e-3) / 1e12,
            "dense_ms": dense_ms,
            "speedup_vs_dense": dense_ms / (g_burst + a_ms),
            "speedup_vs_dense_nomem": dense_ms / a0_ms,
            "theoretical_n_over_tile_plus_region": n / (HILBERT_TILE + G),
            "theoretical_n_over_tile": n / HILBERT_TILE,
        }
        del sets
    res["note"] = ("tile = 256 consecutive Hilbert positions, slide 0 / 128 alternating, "
                   "8x8 central region gathered as memory keys; gather_ms from 20 launches back "
                   "to back between two events (gather_ms_one_launch_events: events around each "
                   "launch); the page's 2.3x (1024^2 px) "
                   "and 4.17x (2048^2 px) are context (its tile and region sizes are not stated)")
    return res


def measure_window(S, wl, args, stream, dev, with_dense=True):
    n, m, G, D, H, B = (wl.n_tokens, wl.window_tokens, wl.mem_tokens, wl.head_dim, wl.heads,
                       wl.batch)
    sets = make_sets(wl, args.sets, dev)
    # per-kernel times from eager steps with events around each kernel; the
    # step time from graph-replayed steps without them
    ms_eager, pool, attn = time_steps(S, wl, sets, args.steps, args.warmup, stream, True)
    try:
        ms_graph, graph_ok = time_steps_graph(S, wl, sets, args.steps, args.warmup, stream, True)
    except Exception as e:  # a runtime without graph capture: report the eager time
        print(f"[bench] graph replay unavailable ({type(e).__name__}: {e}); eager step time",
              file=sys.stderr, flush=True)
        ms_graph, graph_ok = None, False
    ms_step = ms_graph if graph_ok else ms_eager
    flops = window_flops(B, H, n, m, G, D)
    flops_nomem = window_flops(B, H, n, m, 0, D)
    attn_bytes = 4 * B * H * n * D * 2 + 2 * B * H * G * D * 2
    pool_bytes = 2 * B * H * n * D * 2 + 2 * B * H * G * D * 2
    attn_ms = sum(attn) / len(attn)
    pool_ms = sum(pool) / len(pool)
    r = {
        "workload": wl.name, "n": n, "m": m, "G": G,
        "ms_per_step": ms_step,
        "tflops_per_step": flops / (ms_step * 1e-3) / 1e12,
        "step_launch": "hip graph per step" if graph_ok else "eager",
        "graph_output_equals_eager": graph_ok,
        "ms_per_step_eager_with_events": ms_eager,
        "eager_steps_queued_ahead": LAST_TIMING.get("queued_ahead"),
        "ms_per_step_graph": ms_graph,
        "graph_steps_queued_ahead": LAST_TIMING.get("graph_queued_ahead"),
        "window_attn_ms": {"mean": attn_ms, "median": median(attn), "p10": pct(attn, 10),
                           "p90": pct(attn, 90)},
        "pool_kv_ms": {"mean": pool_ms, "median": median(pool)},
        # timed step i runs schedule phase (warmup + i) mod 4
        "window_attn_ms_by_phase": {
            str(ph): sum(a for i, a in enumerate(attn) if (args.warmup + i) % 4 == ph)
            / max(1, sum(1 for i in range(len(attn)) if (args.warmup + i) % 4 == ph))
            for ph in range(4)},
        "window_attn_tflops": flops / (attn_ms * 1e-3) / 1e12,
        "window_attn_mfma_frac": flops / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "window_attn_gbs": attn_bytes / (attn_ms * 1e-3) / 1e9,
        "pool_kv_gbs": pool_bytes / (pool_ms * 1e-3) / 1e9,
        "flops_per_call": flops, "attn_bytes_per_call": attn_bytes,
        "pool_bytes_per_call": pool_bytes,
    }
    # hot cache (secondary): every step on the first input set, so much of
    # Q, K and V (302 MB at FLUX-2048) stays in the 256 MB last-level cache
    ms_hot, pool_hot, attn_hot = time_steps(S, wl, sets[:1], max(10, args.steps // 2), 3, stream,
                                            True)
    r["hot_one_input_set"] = {
        "ms_per_step_eager_with_events": ms_hot,
        "window_attn_ms": sum(attn_hot) / len(attn_hot),
        "pool_kv_ms": sum(pool_hot) / len(pool_hot),
        "window_attn_tflops": flops / (sum(attn_hot) / len(attn_hot) * 1e-3) / 1e12,
    }
    # memory off: the literal n/m comparison
    _, _, attn0 = time_steps(S, wl, sets, max(10, args.steps // 2), 3, stream, False)
    attn0_ms = sum(attn0) / len(attn0)
    r["window_attn_nomem_ms"] = attn0_ms
    r["window_attn_nomem_tflops"] = flops_nomem / (attn0_ms * 1e-3) / 1e12
    if with_dense:
        dense = time_dense(S, sets, args.dense_reps, stream)
        dense_ms = median(dense)
        dflops = dense_flops(B, H, n, D)
        r["dense_ms"] = dense_ms
        r["dense_tflops"] = dflops / (dense_ms * 1e-3) / 1e12
        r["dense_mfma_frac"] = r["dense_tflops"] / PEAK_BF16_TFLOPS
        th_nomem = n / m
        th_mem = n / (m + G)
        r["speedup"] = {
            "theoretical_n_over_m": th_nomem,
            "realised_nomem": dense_ms / attn0_ms,
            "realised_over_theoretical_nomem": dense_ms / attn0_ms / th_nomem,
            "theoretical_n_over_m_plus_G": th_mem,
            "realised_mem": dense_ms / attn_ms,
            "realised_over_theoretical_mem": dense_ms / attn_ms / th_mem,
            "realised_mem_incl_pool": dense_ms / (attn_ms + pool_ms),
        }
    del sets
    return r


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import sparse_window_attention_amd as S
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    head = W.FLUX2048_W16 if args.window == 16 else W.FLUX2048_W32
    other = W.FLUX2048_W32 if args.window == 16 else W.FLUX2048_W16
    print(f"[bench] headline {head.name}: {args.warmup} warmup + {args.steps} timed steps",
          file=sys.stderr, flush=True)
    if args.only == "dense":
        sets = make_sets(head, 1, dev)
        ts = time_dense(S, sets, args.steps, stream)
        print(json.dumps({"dense_ms": median(ts)}))
        return
    if args.only == "copy":
        ts = time_copy(args.steps, stream)
        print(json.dumps({"copy_bytes": COPY_BYTES, "copy_ms": median(ts),
                          "copy_gbs": 2 * COPY_BYTES / (median(ts) * 1e-3) / 1e9}))
        return
    if args.only == "backward":
        sets = make_sets(head, 2, dev)
        print(json.dumps(measure_backward(S, head, sets, args.steps, stream)))
        return
    if args.only == "video":
        runs = {"wan": lambda: measure_other_shape(S, W.WAN, stream, dev, args.steps, 3),
                "wan_g1638": lambda: measure_other_shape(S, W.WAN_G1638, stream, dev,
                                                         args.steps, 3),
                "ultra": lambda: measure_other_shape(S, W.ULTRA, stream, dev,
                                                     max(4, args.steps // 4), 3),
                "flux1024": lambda: measure_other_shape(S, W.FLUX1024, stream, dev,
                                                        args.steps, 5),
                "tiny_f32": lambda: measure_tiny(S, stream, dev, args.steps)}
        print(json.dumps({k: runs[k]() for k in args.shapes.split(",")}))
        return
    if args.only == "profile":
        print(json.dumps(run_profile_workload(S, args.workload, stream, dev)))
        return
    if args.only == "pool":
        print(json.dumps(measure_pool(S, stream, dev, args.steps)))
        return
    if args.only == "calib":
        print(json.dumps(measure_mfma_peak(S, stream)))
        return
    if args.only == "hilbert":
        print(json.dumps(measure_hilbert(S, stream, dev, args.steps)))
        return
    if args.only == "window":
        sets = make_sets(head, args.sets, dev)
        ms, pool, attn = time_steps(S, head, sets, args.steps, args.warmup, stream, True)
        try:
            ms_g, ok = time_steps_graph(S, head, sets, args.steps, args.warmup, stream, True)
        except Exception:
            ms_g, ok = None, False
        print(json.dumps({"ms_per_step": ms_g if ok else ms, "graph_output_equals_eager": ok,
                          "ms_per_step_eager_with_events": ms,
                          "attn_ms": sum(attn) / len(attn), "pool_ms": sum(pool) / len(pool)}))
        return
    res = measure_window(S, head, args, stream, dev)
    print(f"[bench] {head.name}: attn {res['window_attn_ms']['mean']*1e3:.1f} us "
          f"({res['window_attn_tflops']:.0f} TFLOP/s), pool {res['pool_kv_ms']['mean']*1e3:.1f} us",
          file=sys.stderr, flush=True)
    comp_sets = make_sets(head, args.sets, dev)
    comp = measure_composition(S, head, comp_sets, max(10, args.steps // 2), stream)
    del comp_sets
    comp["fused_attention_ms"] = res["window_attn_ms"]["mean"]
    comp["composition_over_fused"] = comp["total"] / res["window_attn_ms"]["mean"]
    print(f"[bench] composition baseline: gather {comp['roll_partition_gather']*1e3:.1f} + "
          f"memory concat {comp['memory_concat']*1e3:.1f} + dense "
          f"{comp['dense_attention']*1e3:.1f} + unpartition "
          f"{comp['unpartition_unroll']*1e3:.1f} us", file=sys.stderr, flush=True)
    bwd_sets = make_sets(head, 2, dev)
    bwd = measure_backward(S, head, bwd_sets, max(8, args.steps // 4), stream)
    del bwd_sets
    print(f"[bench] backward ({head.name}): forward+lse {bwd['forward_with_lse_ms']*1e3:.1f} us, "
          f"backward {bwd['backward_ms']*1e3:.1f} us ({bwd['backward_tflops']:.0f} TFLOP/s)",
          file=sys.stderr, flush=True)
    hil = measure_hilbert(S, stream, dev, max(8, args.steps // 4))
    print("[bench] hilbert tiles: " + ", ".join(
        f"{k} {v['tile_attn_ms']*1e3:.1f} us ({v['speedup_vs_dense']:.2f}x vs dense)"
        for k, v in hil.items() if k != "note"), file=sys.stderr, flush=True)
    wan = measure_other_shape(S, W.WAN, stream, dev, max(8, args.steps // 4), 3)
    wan["pages_context"] = ("up to 4.52x attention speedup on Wan (the pages' own dense baseline "
                            "and hardware, not stated)")
    wan1638 = measure_other_shape(S, W.WAN_G1638, stream, dev, max(8, args.steps // 4), 3)
    ultra = measure_other_shape(S, W.ULTRA, stream, dev, 4, 3)
    flux1024 = measure_other_shape(S, W.FLUX1024, stream, dev, max(8, args.steps // 2), 5)
    tiny = measure_tiny(S, stream, dev, max(8, args.steps // 2))
    print(f"[bench] wan: attn {wan['window_attn_ms']*1e3:.0f} us ({wan['window_attn_tflops']:.0f} "
          f"TFLOP/s), dense {wan['dense_ms']:.2f} ms; ultra: attn {ultra['window_attn_ms']:.2f} ms, "
          f"dense {ultra['dense_ms']:.0f} ms", file=sys.stderr, flush=True)
    res_o = measure_window(S, other, args, stream, dev)
    print(f"[bench] {other.name}: attn {res_o['window_attn_ms']['mean']*1e3:.1f} us "
          f"({res_o['window_attn_tflops']:.0f} TFLOP/s)", file=sys.stderr, flush=True)

    # roofline of the dominant kernel (window attention) on the headline workload
    flops = res["flops_per_call"]
    byts = res["attn_bytes_per_call"]
    t = res["window_attn_ms"]["mean"] * 1e-3
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if flops / byts >= ridge:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = "attn_bf16_persistent_kernel<128,false,8,64,true>"
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = byts
    roof["mfma_frac"] = res["window_attn_mfma_frac"]
    calib = measure_mfma_peak(S, stream)
    roof["measured_mfma_peak_tflops"] = calib["tflops"]
    roof["frac_of_measured_mfma_peak"] = flops / t / 1e12 / calib["tflops"]
    roof["kernel_source_hash"] = kernel_hash()
    if os.path.exists(TRAFFIC_FILE):
        try:
            tr = json.load(open(TRAFFIC_FILE))
            if tr.get("kernel_source_hash") == roof["kernel_source_hash"] and \
                    tr.get("workload") == head.name:
                roof["traffic"] = tr["hbm_bytes_per_launch"]
        except Exception:
            pass

    line = {
        "metric": "ms/attn call + effective TFLOP/s (MFMA util) at FLUX-2048 shape; "
                  "realised/theory speedup",
        "value": res["tflops_per_step"],
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head.name, "global_batch": head.batch, "seq_len": head.n_tokens,
                   "heads": head.heads, "head_dim": head.head_dim, "grid": list(head.grid),
                   "window": list(head.window), "pool": list(head.pool),
                   "mem_tokens": head.mem_tokens, "schedule": "four-phase",
                   "input_sets_rotated": args.sets, "step_launch": res["step_launch"],
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "ms_per_attn_call": res["window_attn_ms"]["mean"],
        "windows": {f"{res['m']}": res, f"{res_o['m']}": res_o},
        "composition_baseline": comp,
        "backward": bwd,
        "hilbert_tiles": hil,
        "mfma_calibration": calib,
        "other_shapes": {"flux1024": flux1024, "wan": wan, "wan_g1638": wan1638,
                         "ultra": ultra, "tiny_f32": tiny},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(head, args.cpu_seconds)
        line["cpu_baseline"]["other_configs"] = oracle_per_config()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
