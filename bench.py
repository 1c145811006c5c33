#!/usr/bin/env python3
"""Benchmark: batched speculative-sampling verification on one MI355X.

A step is one sv_verify call over one batch of a synthetic workload (every
kernel of the hot path: softmax statistics, acceptance ratios, first-rejection
ballot, residual / bonus Gumbel-max sampling).  Inputs are resident in HBM
before timing starts; at least two copies are rotated, more when the rows a
step surely reads (position 0) come to less than 1 GiB over two, so a step
does not find rows an earlier step left in the 256 MB last-level cache
(workloads whose whole input is far smaller, like c1, still fit it).

Prints ONE JSON line: verified draft positions per second on the headline
workload (c4b: B=1024, gamma=4, V=50257, fp32, draft noise sigma 1), the
roofline of the dominant kernel measured with HIP events recorded by the
library around each launch, the CPU oracle timed on a bounded sample on this
host, and the same measurements for the other workloads under "sweep".
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
HEADLINE = "c4b"
SWEEP = ["c2", "c3", "c3p", "c2p", "c4a", "c4c", "c1", "g4b", "g2"]
PROFILE_DIR = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rejection_sampling_verify_17_amd", "csrc")


# ---------------------------------------------------------------------------
# HIP events (the library records them on the caller's stream)
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.L = ctypes.CDLL("libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = ctypes.c_void_p()
        assert self.L.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, stream) == 0

    def sync(self, e):
        assert self.L.hipEventSynchronize(e) == 0

    def ms(self, a, b) -> float:
        f = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return float(f.value)

    def destroy(self, e):
        self.L.hipEventDestroy(e)


def source_digest() -> str:
    """Digest of the kernel sources with comments and blank space removed, so
    that counter summaries stay valid across edits of the documentation only."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = " ".join(text.split())
        h.update(f.encode() + b"\0" + text.encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Algorithmic bytes
# ---------------------------------------------------------------------------
def algorithmic_bytes(w, n_accepted: np.ndarray) -> dict:
    """Bytes the method must move, from the step's own
    outcome n_b.  The drafts are judged left to right and nothing after the
    first rejection is needed, so the statistics read row pairs 0..n_b
    (min(n_b + 1, gamma) pairs, 2 V b bytes each); the resample then reads
    row pair n_b again (2 V b; with top-k it works from the kept lists
    instead) or the bonus row (V b).  Plus tokens in and outputs out.  In the
    arg-max mode (T = 0) only target rows 0..n_b are needed, once each."""
    B, gamma, V = w.B, w.gamma, w.V
    b = 2 if w.is_bf16 else 4
    n = n_accepted[n_accepted >= 0].astype(np.int64)
    io = 4 * B * gamma + 4 * B * (gamma + 1) + 4 * B
    if w.temperature == 0.0:
        # arg-max mode: target rows 0..n_b, once each (the last one holds the token)
        rows = int(np.sum(n + 1)) * V * b
        return {"stats": rows, "sample": 0, "io": io, "total": rows + io,
                "all_rows_once": B * (gamma + 1) * V * b}
    stats = int(np.sum(np.minimum(n + 1, gamma))) * 2 * V * b
    rej = int(np.sum(n < gamma))
    bonus = int(np.sum(n == gamma))
    sample = (0 if 0 < w.top_k < V else rej * 2 * V * b) + bonus * V * b
    all_rows = 2 * B * gamma * V * b  # every draft and target row 0..gamma-1 once
    return {"stats": stats, "sample": sample, "io": io, "total": stats + sample + io,
            "all_rows_once": all_rows}


# ---------------------------------------------------------------------------
# One workload
# ---------------------------------------------------------------------------
def run_workload(name: str, steps: int, warmup: int, hip: Hip, seed: int = 3000) -> dict:
    import torch
    import rejection_sampling_verify_17_amd as S
    from workloads import synth as I

    t0 = time.time()
    w = I.make(name)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")
    # copies enough that the rows a step surely reads (position 0: the target
    # row, and the draft row unless T = 0) add up to 1 GiB over the rotation,
    # so the 256 MB MALL cannot serve a repeat (capped at 8 copies)
    first = (1 if w.temperature == 0.0 else 2) * w.B * w.V * (2 if w.is_bf16 else 4)
    copies = max(2, min(8, int(np.ceil((1 << 30) / first))))
    if w.is_bf16:
        tgt0 = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16)
        drf0 = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16)
    else:
        tgt0, drf0 = torch.from_numpy(w.target), torch.from_numpy(w.draft)
    tgts = [tgt0.to(dev) for _ in range(copies)]
    drfs = [drf0.to(dev) for _ in range(copies)]
    tok = torch.from_numpy(w.tokens).to(dev)
    dt = S.SV_BF16 if w.is_bf16 else S.SV_F32
    ws = torch.zeros(S.workspace_bytes(w.B, w.gamma, w.V, w.top_k, dt), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.gamma + 1), dtype=torch.int32, device=dev)
    nacc = torch.empty((w.B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    names = S.launch_names(w.B, w.gamma, w.V, dt, w.top_k, w.temperature, w.top_p)
    nl = len(names)

    def step(i, events=None):
        k = i % copies
        if events is None:
            S.verify(tgts[k], drfs[k], tok, w.temperature, w.top_k, seed=seed, out_tokens=out, n_accepted=nacc,
                     workspace=ws, top_p=w.top_p)
        else:
            S.verify_timed(tgts[k], drfs[k], tok, w.temperature, events, w.top_k, seed=seed, out_tokens=out,
                           n_accepted=nacc, workspace=ws, top_p=w.top_p)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: plain calls bracketed by events on the launch stream.
    e0, e1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(e0, sp)
    for i in range(steps):
        step(i)
    hip.record(e1, sp)
    hip.sync(e1)
    torch.cuda.synchronize()
    ms_total = hip.ms(e0, e1)
    ms_step = ms_total / steps

    # Same steps again with the library recording an event pair around each
    # kernel: per-kernel average durations for the roofline.
    evs = [[hip.event() for _ in range(2 * nl)] for _ in range(steps)]
    f0, f1 = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(f0, sp)
    for i in range(steps):
        step(i, evs[i])
    hip.record(f1, sp)
    hip.sync(f1)
    torch.cuda.synchronize()
    per_kernel = {}
    for kname in dict.fromkeys(names):
        idx = [li for li, nm in enumerate(names) if nm == kname]
        per_step = [sum(hip.ms(evs[i][2 * li], evs[i][2 * li + 1]) for li in idx) for i in range(steps)]
        per_kernel[kname] = {"launches_per_step": len(idx), "us_per_step": 1e3 * float(np.mean(per_step)),
                             "avg_us": 1e3 * float(np.mean(per_step)) / len(idx),
                             "min_step_us": 1e3 * float(np.min(per_step))}
    ms_step_evented = hip.ms(f0, f1) / steps
    for row in evs:
        for e in row:
            hip.destroy(e)
    for e in (e0, e1, f0, f1):
        hip.destroy(e)

    n_acc = nacc.cpu().numpy()
    out_np = out.cpu().numpy()
    ab = algorithmic_bytes(w, n_acc)
    positions = w.B * w.gamma
    # the kernel that takes most of the step (every byte of the rows goes through it)
    dominant = max(per_kernel, key=lambda k: per_kernel[k]["us_per_step"])
    dom_launches = per_kernel[dominant]["launches_per_step"]
    dom_bytes = ab["stats"] + ab["sample"] + 4 * w.B * w.gamma
    dom_us = per_kernel[dominant]["avg_us"]
    res = {
        "workload": name, "B": w.B, "gamma": w.gamma, "V": w.V, "dtype": "bf16" if w.is_bf16 else "f32",
        "temperature": w.temperature, "top_k": w.top_k, "top_p": w.top_p, "input_copies": copies,
        "ms_per_step": ms_step, "ms_per_step_with_kernel_events": ms_step_evented,
        "positions_per_s": positions / (ms_step * 1e-3),
        "algorithmic_bytes": ab, "GBps_step": ab["total"] / (ms_step * 1e-3) / 1e9,
        "frac_peak_step": ab["total"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels": per_kernel, "dominant": dominant,
        "dominant_GBps": dom_bytes / (dom_us * dom_launches * 1e-6) / 1e9,
        "dominant_bytes_per_launch": dom_bytes / dom_launches, "dominant_launches": dom_launches,
        "mean_accepted": float(n_acc[n_acc >= 0].mean()), "all_kept": float(np.mean(n_acc == w.gamma)),
        "gen_s": gen_s,
    }
    del tgts, drfs
    torch.cuda.empty_cache()
    return res, w, (out_np, n_acc)


# ---------------------------------------------------------------------------
# Draft-token sampling (the step before verification)
# ---------------------------------------------------------------------------
def run_draft(name: str, steps: int, warmup: int, hip: Hip, seed: int = 3000) -> dict:
    """sv_draft_sample over the draft rows of a workload: every row read once,
    one Philox word and two logarithms per entry (no top-k)."""
    import torch
    import rejection_sampling_verify_17_amd as S
    from workloads import synth as I
    w = I.make(name)
    dev = torch.device("cuda:0")
    copies = max(2, min(8, int(np.ceil((1 << 30) / w.draft.nbytes))))
    if w.is_bf16:
        d0 = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16)
    else:
        d0 = torch.from_numpy(w.draft)
    drfs = [d0.to(dev) for _ in range(copies)]
    out = torch.empty((w.B, w.gamma), dtype=torch.int32, device=dev)
    sp = int(torch.cuda.current_stream(dev).cuda_stream)
    for i in range(warmup):
        S.draft_sample(drfs[i % copies], w.temperature, w.top_k, seed=seed, out=out, top_p=w.top_p)
    torch.cuda.synchronize()
    e0, e1 = hip.event(), hip.event()
    hip.record(e0, sp)
    for i in range(steps):
        S.draft_sample(drfs[i % copies], w.temperature, w.top_k, seed=seed, out=out, top_p=w.top_p)
    hip.record(e1, sp)
    hip.sync(e1)
    us = hip.ms(e0, e1) / steps * 1e3
    hip.destroy(e0)
    hip.destroy(e1)
    rows = w.B * w.gamma
    nbytes = w.draft.nbytes + 4 * rows
    return {"workload": f"{name} draft rows", "kernel": "k_draft_sample", "us_per_call": us,
            "drafted_tokens_per_s": rows / (us * 1e-6), "GBps": nbytes / (us * 1e-6) / 1e9,
            "entries_per_s": rows * w.V / (us * 1e-6)}


# ---------------------------------------------------------------------------
# Traffic from committed rocprofv3 PMC summaries
# ---------------------------------------------------------------------------
def read_traffic(kernel: str, workload: str) -> float | None:
    """HBM bytes per launch from profiles/<kernel>_<workload>_pmc.txt, or None if
    absent or taken on different kernel sources."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline(w, seed: int, budget_s: float = 12.0, gpu_out=None) -> dict:
    """The oracle as it stands on this host's cores, on a bounded sample: the
    first n sequences of the workload (n sized so one run takes about
    budget_s / 3; all B if they fit, the batch then repeated under as many
    verify seeds as fill that time), one warm-up run, then the median of 3
    timed runs, in verified positions per second.  Its outputs (verify seed
    `seed`, the seed the timed GPU steps used) are compared with the GPU's
    outputs for the same sequences (`gpu_out` = (out_tokens, n_accepted) of
    the last timed step) under the parity bar of tests/parity.py."""
    from oracle import oracle as O
    cores = len(os.sched_getaffinity(0))
    B = w.B
    target_s = budget_s / 3.0
    n = min(B, max(cores, 8))
    t0 = time.perf_counter()
    O.verify(w.target[:n], w.draft[:n], w.tokens[:n], w.temperature, w.top_k, seed=seed, nthreads=cores,
             top_p=w.top_p)
    t1 = time.perf_counter() - t0
    if t1 < target_s / 2 and n < B:
        n = int(min(B, max(n + 1, n * (target_s / max(t1, 1e-3)))))
    t0 = time.perf_counter()
    O.verify(w.target[:n], w.draft[:n], w.tokens[:n], w.temperature, w.top_k, seed=seed, nthreads=cores,
             top_p=w.top_p)  # warm-up at the final size
    t1 = time.perf_counter() - t0
    # when the whole batch takes less, a run repeats it under further verify seeds
    reps = max(1, int(round(target_s / max(t1, 1e-3)))) if n == B else 1
    times = []
    for r in range(3):
        t0 = time.perf_counter()
        for k in range(reps):
            O.verify(w.target[:n], w.draft[:n], w.tokens[:n], w.temperature, w.top_k, seed=seed + r * reps + k,
                     nthreads=cores, top_p=w.top_p)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    res = {"value": n * w.gamma * reps / t, "unit": "verified draft positions/s", "cores": cores,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"first {n} of {B} sequences of {w.spec.name}, {reps} verify seed(s) per run "
                     f"(seeds {seed}..{seed + 3 * reps - 1}), median of 3 runs "
                     f"({', '.join(f'{x:.2f}' for x in times)} s) on {cores} threads"}
    if gpu_out is not None:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        try:
            import parity as PT
        finally:
            sys.path.pop(0)
        from workloads import synth as I
        ws = I.from_arrays(w.target[:n], w.draft[:n], w.tokens[:n], w.temperature, w.top_k, top_p=w.top_p)
        g = PT.GpuResult(gpu_out[0][:n], gpu_out[1][:n])
        rep = PT.compare(ws, seed, g, nthreads=cores, check_probs=False)
        sm = rep.summary()
        res["parity_of_timed_outputs"] = {k: sm[k] for k in ("sequences", "mismatches", "exempt_accept",
                                                             "exempt_token", "exempt_nucleus", "exempt_equal")}
    return res


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_one_thread(name: str = "c2", n: int = 4, seed: int = 3000) -> dict:
    """The oracle on one host thread, the first n sequences of a workload: a
    per-core figure beside the all-core baseline."""
    from oracle import oracle as O
    from workloads import synth as I
    w = I.make(name, B=n)
    t0 = time.perf_counter()
    O.verify(w.target, w.draft, w.tokens, w.temperature, w.top_k, seed=seed, nthreads=1, top_p=w.top_p)
    t = time.perf_counter() - t0
    return {"workload": name, "sequences": n, "seconds": t, "positions_per_s": n * w.gamma / t, "threads": 1}


def stream_read_GBps(hip: Hip, gib: int = 1) -> dict:
    """Context only: the read rate of a plain streaming kernel of the library
    (sv_probe_read: contiguous slabs, four 16-byte loads in flight per
    thread; with ordinary and with non-temporal loads) over `gib` GiB, per
    grid size, mean of 10 launches timed by HIP events on the launch stream;
    and, for comparison, torch.sum over the same buffer."""
    import torch
    import rejection_sampling_verify_17_amd as S
    nbytes = gib << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    out = torch.empty(65536, dtype=torch.float32, device="cuda")
    sp = int(torch.cuda.current_stream().cuda_stream)
    e0, e1 = hip.event(), hip.event()
    rates, rates_nt = {}, {}
    for nt, dst in ((0, rates), (1, rates_nt)):
        for grid in (1024, 2048, 4096, 8192, 16384):
            for _ in range(3):
                assert S.lib().sv_probe_read(x.data_ptr(), nbytes, out.data_ptr(), grid, nt, sp) == 0
            hip.record(e0, sp)
            for _ in range(10):
                S.lib().sv_probe_read(x.data_ptr(), nbytes, out.data_ptr(), grid, nt, sp)
            hip.record(e1, sp)
            hip.sync(e1)
            dst[str(grid)] = nbytes * 10 / (hip.ms(e0, e1) * 1e-3) / 1e9
    for _ in range(3):
        x.sum()  # warm-up: the first call also loads the reduction kernel
    torch.cuda.synchronize()
    hip.record(e0, sp)
    for _ in range(10):
        x.sum()
    hip.record(e1, sp)
    hip.sync(e1)
    torch_sum = nbytes * 10 / (hip.ms(e0, e1) * 1e-3) / 1e9
    hip.destroy(e0)
    hip.destroy(e1)
    del x, out
    torch.cuda.empty_cache()
    return {"probe_read_GBps_by_grid": rates, "probe_read_GBps_best": max(rates.values()),
            "probe_read_nontemporal_GBps_by_grid": rates_nt,
            "probe_read_nontemporal_GBps_best": max(rates_nt.values()),
            "torch_sum_GBps": torch_sum, "bytes": nbytes}


# ---------------------------------------------------------------------------
# rocprofv3 CSV -> short text summaries (what profiles/ holds)
# ---------------------------------------------------------------------------
def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    out = []
    for root, _, files in os.walk(d):
        out += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    return sorted(out)


def _short(name: str) -> str:
    for k in ("k_topk_step", "k_greedy_step", "k_draft_sample", "k_accept_hist", "k_rows", "k_judge"):
        if k in name:
            return k
    return name[:60]


def kernel_stats_summary(d: str) -> list[str]:
    lines = ["kernel | calls | avg_us | min_us | max_us | total_us | percent"]
    for path in _find(d, "kernel_stats.csv"):
        for r in _csv_rows(path):
            lines.append(f"{_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.2f}")
    return lines


def counter_means(d: str) -> dict:
    """{(kernel short name, counter): (mean per dispatch, dispatches)} from counter_collection.csv."""
    acc = {}
    for path in _find(d, "counter_collection.csv"):
        for r in _csv_rows(path):
            key = (_short(r["Kernel_Name"]), r["Counter_Name"])
            acc.setdefault(key, {})
            disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
            acc[key][disp] = acc[key].get(disp, 0.0) + float(r["Counter_Value"])
    return {k: (float(np.mean(list(v.values()))), len(v)) for k, v in acc.items()}


def rocprof_summary(args) -> None:
    """Summaries for profiles/: --rocprof-summary DIR with sub-directories
    trace/ (kernel trace + stats), fetch/ and write/ (FETCH_SIZE, WRITE_SIZE on
    the workload), cfetch/ and cwrite/ (the same counters on a plain copy of
    --copy-calib-mb MiB)."""
    d = args.rocprof_summary
    wl = args.workload
    out = []
    out.append(f"# rocprofv3 kernel trace, workload {wl}")
    extra = "--draft-only" if args.draft_only else "--no-cpu --no-sweep"
    out.append(f"command: rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/trace -o run -- "
               f"python3 bench.py --workload {wl} --steps {args.steps} --warmup {args.warmup} {extra}")
    out.append(f"source_digest: {source_digest()}")
    out += kernel_stats_summary(os.path.join(d, "trace"))
    with open(os.path.join(d, f"kernel_trace_{wl}{'_draft' if args.draft_only else ''}.txt"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))
    fetch = counter_means(os.path.join(d, "fetch"))
    write = counter_means(os.path.join(d, "write"))
    cf = counter_means(os.path.join(d, "cfetch"))
    cw = counter_means(os.path.join(d, "cwrite"))
    if not (fetch and write and cf and cw):
        print("no counter data")
        return
    copy_bytes = args.copy_calib_mb << 20

    def copy_factor(means, counter):
        vals = [(v, n) for (k, c), (v, n) in means.items() if c == counter and "copy" in k.lower()]
        if not vals:
            vals = [(v, n) for (k, c), (v, n) in means.items() if c == counter]
        v = max(vals)[0]
        return copy_bytes / (v * 1024.0), v

    ff, fv = copy_factor(cf, "FETCH_SIZE")
    wf, wv = copy_factor(cw, "WRITE_SIZE")
    for (k, c), (v, n) in sorted(fetch.items()):
        if c != "FETCH_SIZE" or not k.startswith("k_"):
            continue
        wkib = write.get((k, "WRITE_SIZE"), (0.0, 0))[0]
        hbm = v * 1024.0 * ff + wkib * 1024.0 * wf
        lines = [f"# HBM traffic of {k}, workload {wl}",
                 f"command: rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- python3 bench.py "
                 f"--workload {wl} --steps {args.steps} --warmup {args.warmup} {extra} ; the same with "
                 f"--pmc WRITE_SIZE ; and both counters on: python3 bench.py --copy-calib-mb {args.copy_calib_mb}",
                 f"source_digest: {source_digest()}",
                 f"dispatches: {n}",
                 f"fetch_kib_per_launch: {v:.1f}",
                 f"write_kib_per_launch: {wkib:.1f}",
                 f"copy_calib_bytes: {copy_bytes}",
                 f"copy_fetch_kib: {fv:.1f}",
                 f"copy_write_kib: {wv:.1f}",
                 f"fetch_scale: {ff:.4f}",
                 f"write_scale: {wf:.4f}",
                 f"hbm_bytes_per_launch: {hbm:.0f}"]
        with open(os.path.join(d, f"{k}_{wl}_pmc.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines))


def _kernel_variant(name: str) -> str:
    """Kernel name with its template arguments (e.g. k_rows<1, 0>), else the short name."""
    short = _short(name)
    i = name.find(short + "<")
    if i >= 0:
        j = name.find(">", i)
        if j > 0:
            return name[i:j + 1]
    return short


def busy_summary(args) -> None:
    """Summary for profiles/ of one rocprofv3 --pmc run under --rocprof-busy DIR
    (sub-directory busy/) with VALUBusy, TA_BUSY_avr, SQ_INSTS_VALU,
    SQ_INSTS_VALU_TRANS_F32 and GRBM_GUI_ACTIVE: per kernel instantiation, the
    mean over its dispatches of the VALU-busy percentage (rocprofv3's derived
    VALUBusy), the memory-unit (texture addresser) busy percentage
    TA_BUSY_avr / GRBM_GUI_ACTIVE, and the VALU and transcendental
    instructions per dispatch."""
    d = args.rocprof_busy
    wl = args.workload
    acc = {}
    for path in _find(os.path.join(d, "busy"), "counter_collection.csv"):
        for r in _csv_rows(path):
            key = _kernel_variant(r["Kernel_Name"])
            disp = r.get("Dispatch_Id") or r.get("Correlation_Id")
            acc.setdefault(key, {}).setdefault(disp, {})
            c = r["Counter_Name"]
            acc[key][disp][c] = acc[key][disp].get(c, 0.0) + float(r["Counter_Value"])
    extra = "--no-cpu --no-sweep"
    lines = [f"# VALU and memory-unit busy, workload {wl}",
             f"command: rocprofv3 --pmc VALUBusy TA_BUSY_avr SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE "
             f"--output-format csv -d <dir>/busy -o run -- python3 bench.py --workload {wl} --steps {args.steps} "
             f"--warmup {args.warmup} {extra}",
             f"source_digest: {source_digest()}",
             "kernel | dispatches | VALU busy % | memory unit busy % | VALU instructions | transcendental instructions"]
    for k, disps in sorted(acc.items()):
        if not k.startswith("k_"):
            continue
        vb = [v.get("VALUBusy", np.nan) for v in disps.values()]
        mb = [100.0 * v.get("TA_BUSY_avr", np.nan) / v["GRBM_GUI_ACTIVE"]
              for v in disps.values() if v.get("GRBM_GUI_ACTIVE")]
        vi = [v.get("SQ_INSTS_VALU", np.nan) for v in disps.values()]
        ti = [v.get("SQ_INSTS_VALU_TRANS_F32", np.nan) for v in disps.values()]
        lines.append(f"{k} | {len(disps)} | {np.nanmean(vb):.1f} | {np.nanmean(mb):.1f} | "
                     f"{np.nanmean(vi):.4g} | {np.nanmean(ti):.4g}")
    with open(os.path.join(d, f"busy_{wl}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    ap.add_argument("--draft-only", action="store_true",
                    help="only time draft-token sampling on the workload's draft rows and print its JSON")
    ap.add_argument("--rocprof-summary", metavar="DIR", default=None,
                    help="summarise rocprofv3 CSV output under DIR (see rocprof_summary) and exit")
    ap.add_argument("--rocprof-busy", metavar="DIR", default=None,
                    help="summarise a rocprofv3 busy-counter run under DIR/busy (see busy_summary) and exit")
    args = ap.parse_args()
    if args.rocprof_busy:
        busy_summary(args)
        return
    if args.rocprof_summary:
        rocprof_summary(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the library is measured on one GPU only; run with --gpus 1"}))
        sys.exit(2)

    import torch
    if args.copy_calib_mb:
        n = args.copy_calib_mb << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    import rejection_sampling_verify_17_amd as S
    S.lib()
    hip = Hip()
    if args.draft_only:
        print(json.dumps(run_draft(args.workload, args.steps, args.warmup, hip)))
        return
    print(f"# bench {args.workload}: steps {args.steps} warmup {args.warmup}", file=sys.stderr, flush=True)
    head, w, head_out = run_workload(args.workload, args.steps, args.warmup, hip)
    print(f"# {args.workload}: {head['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
    dom = head["dominant"]
    dom_us = head["kernels"][dom]["avg_us"]
    traffic = read_traffic(dom, args.workload)
    roofline = {"bound": "hbm", "kernel": dom, "achieved": head["dominant_GBps"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": head["dominant_GBps"] / HBM_PEAK_GBS, "traffic": traffic,
                "algorithmic_bytes_per_launch": head["dominant_bytes_per_launch"], "avg_launch_us": dom_us,
                "launches_per_step": head["dominant_launches"]}
    cpu = None if args.no_cpu else cpu_baseline(w, 3000, budget_s=15.0, gpu_out=head_out)
    if cpu is not None:
        cpu["one_thread"] = cpu_one_thread()
        print(f"# cpu baseline {args.workload}: {cpu['value']:.0f} positions/s; timed-output parity "
              f"{cpu.get('parity_of_timed_outputs')}", file=sys.stderr, flush=True)
    sweep = []
    if not args.no_sweep:
        for name in SWEEP:
            if name == args.workload:
                continue
            r, wr, rout = run_workload(name, max(10, args.steps // 2), max(3, args.warmup // 2), hip)
            print(f"# {name}: {r['ms_per_step'] * 1e3:.1f} us/step", file=sys.stderr, flush=True)
            entry = {k: r[k] for k in ("workload", "ms_per_step", "positions_per_s", "GBps_step",
                                       "frac_peak_step", "dominant", "dominant_GBps", "kernels",
                                       "mean_accepted", "input_copies")}
            entry["roofline"] = {"bound": "hbm", "kernel": r["dominant"], "achieved": r["dominant_GBps"],
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": r["dominant_GBps"] / HBM_PEAK_GBS,
                                 "traffic": read_traffic(r["dominant"], name),
                                 "algorithmic_bytes_per_launch": r["dominant_bytes_per_launch"],
                                 "avg_launch_us": r["kernels"][r["dominant"]]["avg_us"],
                                 "launches_per_step": r["dominant_launches"]}
            if not args.no_cpu:
                entry["cpu_baseline"] = cpu_baseline(wr, 3000, budget_s=3.0, gpu_out=rout)
                print(f"# cpu baseline {name}: {entry['cpu_baseline']['value']:.0f} positions/s; parity "
                      f"{entry['cpu_baseline'].get('parity_of_timed_outputs')}", file=sys.stderr, flush=True)
            sweep.append(entry)
    draft = None
    if not args.no_sweep:
        draft = run_draft(HEADLINE, max(30, args.steps // 2), max(40, args.warmup), hip)
        print(f"# draft sampling {HEADLINE}: {draft['us_per_call']:.1f} us/call", file=sys.stderr, flush=True)
    line = {
        "metric": "verified draft positions/sec (and HBM GB/s, fraction of MI355X peak) at 1 GPU",
        "value": head["positions_per_s"], "unit": "verified draft positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if not w.is_bf16 else "bf16", "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={w.B} gamma={w.gamma} V={w.V} "
                               f"{'bf16' if w.is_bf16 else 'fp32'} T={w.temperature} top_k={w.top_k}",
                   "B": w.B, "gamma": w.gamma, "V": w.V, "parallelism": "single GPU"},
        "GBps_step": head["GBps_step"], "frac_peak_step": head["frac_peak_step"],
        "kernels": head["kernels"], "mean_accepted": head["mean_accepted"],
        "roofline": roofline, "cpu_baseline": cpu, "sweep": sweep, "draft_sampling": draft,
        "context": {"read_stream": None if args.no_sweep else stream_read_GBps(hip)},
        "source_digest": source_digest(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
