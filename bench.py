#!/usr/bin/env python3
"""Benchmark of the GIE zonal scatter hot path on one MI355X.

One step = one pass of the whole path over one frame of synthetic input that
is already resident in HBM: the stable destination CSR build, the fused
forward and the fused backward (zs_build_csr in its asynchronous mode, so the
step has no host synchronization, then zs_forward and zs_backward), all on
torch's current stream.  W warmup steps, then exactly K timed steps between
two device synchronizations.  HIP events recorded on the same stream bracket
the build and the forward + backward pair of every timed step; K more steps
with an extra event between forward and backward give the per-call durations
(an event between the two calls costs a few microseconds of its own, so it is
kept out of the pair's timing).

The JSON line's ``value`` is the algorithmic HBM throughput of forward +
backward (GB/s): the unique bytes those two calls must move, divided by their
mean event-timed duration.  The headline workload is the 4096-atom frame:
N = 4096 nodes, E = 647170 edges, C = 32 channels, fp32.

The ``cpu_baseline`` leg times the CPU oracle (single-threaded plain C) on
the same inputs.  ``copy_probe`` times a plain 256 MiB device copy in the same
run, for context.  ``flushed`` times forward + backward with the caches
emptied first by reading a 512 MiB buffer (clean lines, no write-back inside
the sample), ``flushed_fill`` the same after overwriting it instead.

The fresh-process protocol runs by default (``--processes 3``; 0 skips it):
before this process touches the GPU, N child processes each run 12 warmup
steps and 50 samples of (build, forward, backward) with per-call events, with
the caches flushed before each sample (read flush, then fill flush) and
without; ``protocol`` reports the median of the per-process medians.  Its
``flushed`` figure is the cold-cache headline.  ``workloads`` adds the warm
and flushed forward + backward of the 1000-node, skewed and 16384-node
frames.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import statistics
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic  # noqa: E402

METRIC = "zonal scatter fwd+bwd µs and HBM GB/s (% peak) at N=4096,E=647170,C=32"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published peak
COPY_CALIBRATION_BYTES = 256 * 1024 * 1024   # bytes read (and written) by the calibration copy
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_headline.json")
_CSRC = os.path.join(ROOT, "edge_node_scatter_amd", "csrc")
# Sources that determine each kernel family's code (compiler flags live in build.py).
KERNEL_SOURCES = {
    "fwd": ["zs_fwd.hip", "zs_internal.h"],
    "bwd": ["zs_bwd.hip", "zs_internal.h"],
    "csr": ["zs_csr.hip", "zs_csr.h", "zs_internal.h"],
    "norm": ["zs_norm.hip", "zs_internal.h"],
}


def algorithmic_bytes(n_edges: int, n_nodes: int, channels: int) -> dict:
    """Unique bytes each call must move (fp32 data, int32 indices).

    forward : per edge coupling 15*4 + radial 3*C*4 + perm 4; per node
              rowptr 4 + out 16*C*4 (plus one rowptr entry)
    backward: per edge 2*(15*4 + 3*C*4) (read both operands, write both
              gradients) + 4 for its edge index; per node grad_out 16*C*4
    build   : per edge dst read twice (2*8) + perm and dst32 written (2*4);
              per node rowptr 4 (plus one entry)
    """
    E, N, C = n_edges, n_nodes, channels
    fwd = E * (15 * 4 + 3 * C * 4 + 4) + (N + 1) * 4 + N * 16 * C * 4
    bwd = E * (2 * (15 * 4 + 3 * C * 4) + 4) + N * 16 * C * 4
    build = E * (2 * 8 + 2 * 4) + (N + 1) * 4
    return {"fwd": fwd, "bwd": bwd, "build": build}


def algorithmic_bytes_normalized(n_edges: int, n_nodes: int, channels: int) -> dict:
    """Unique bytes of the calls with the fused degree normalisation.

    forward : the plain forward's bytes + env 4 per edge + y 16*C*4 and
              norm 4 per node (out is still written: the backward needs it)
    backward: the plain backward's bytes (grad_y takes grad_out's place) +
              per node out rows 1..15 (15*C*4), norm 4 and grad_deg 4; per edge
              dst32 4 and grad_env 4
    """
    E, N, C = n_edges, n_nodes, channels
    b = algorithmic_bytes(E, N, C)
    return {"fwd": b["fwd"] + 4 * E + N * (16 * C * 4 + 4),
            "bwd": b["bwd"] + N * (15 * C * 4 + 8) + 8 * E}


def _code_only(text: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed (so that
    editing a comment does not invalidate counter data taken on the code)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(family: str | None = None) -> str:
    """Hash of the code (comments and whitespace ignored) of one kernel
    family's sources, or of all, and of the build flags."""
    files = sorted({f for fam, fs in KERNEL_SOURCES.items() if family in (None, fam) for f in fs})
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(_CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    with open(os.path.join(_CSRC, "..", "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _family(kernel: str) -> str:
    for fam in ("fwd", "bwd", "norm"):
        if fam in kernel:
            return fam
    return "csr"


def load_traffic(kernel: str, n_calls_per_step: int = 1):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != kernel_source_hash(_family(kernel)):
        return None
    return k.get("hbm_bytes_per_launch")


def _kernel_short_name(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def write_traffic(fetch_csv: str, write_csv: str, out_path: str | None = None) -> dict:
    """Per-kernel HBM bytes per launch from two rocprofv3 --pmc runs of
    ``bench.py --calibrate-copy`` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch), each scaled by what the same counter reads for the plain
    256 MiB device copy of the same run.  Writes profiles/traffic_headline.json
    (or out_path) and returns it."""
    import csv
    import collections

    def per_kernel(path, counter):
        vals = collections.defaultdict(list)
        copies = []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                kib = float(r["Counter_Value"])
                name = _kernel_short_name(r["Kernel_Name"])
                if "copyBuffer" in name and kib > COPY_CALIBRATION_BYTES / 1024 / 8:
                    copies.append(kib)
                elif name.startswith("zs::"):
                    vals[name].append(kib)
        if not copies:
            raise RuntimeError(f"{path}: no calibration copy found")
        scale = (COPY_CALIBRATION_BYTES / 1024) / statistics.median(copies)
        return {k: statistics.fmean(v) for k, v in vals.items()}, scale, copies

    fetch, fscale, fcopies = per_kernel(fetch_csv, "FETCH_SIZE")
    write, wscale, wcopies = per_kernel(write_csv, "WRITE_SIZE")
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        fb = fetch.get(name, 0.0) * 1024 * fscale
        wb = write.get(name, 0.0) * 1024 * wscale
        key = name.split("::")[-1].split("<")[0]
        kernels.setdefault(key, {})[name] = {
            "source_hash": kernel_source_hash(_family(key)),
            "fetch_kib_raw": round(fetch.get(name, 0.0), 1),
            "write_kib_raw": round(write.get(name, 0.0), 1),
            "fetch_bytes": round(fb), "write_bytes": round(wb),
            "hbm_bytes_per_launch": round(fb + wb)}
    out = {"fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
           "calibration_copy_bytes": COPY_CALIBRATION_BYTES,
           "calibration_fetch_kib_raw": fcopies, "calibration_write_kib_raw": wcopies,
           "kernels": {k: (list(v.values())[0] if len(v) == 1 else v) for k, v in kernels.items()}}
    with open(out_path or TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def kernel_roofline(kernel: str, alg_bytes: int, avg_us: float, headline: bool) -> dict:
    """Algorithmic bytes per launch over the mean per-call event time, against
    the HBM peak; ``traffic`` is the committed counter figure (HBM bytes per
    launch) for the headline frame while the kernel's sources are unchanged."""
    gbs = alg_bytes / (avg_us * 1e-6) / 1e9
    traffic = load_traffic(kernel) if headline else None
    return {"avg_launch_us": round(avg_us, 2), "algorithmic_bytes_per_launch": alg_bytes,
            "achieved_gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / alg_bytes, 3) if traffic else None}


def summarize_counters(paths: list[str]) -> dict:
    """Mean value per dispatch of every counter, per zs:: kernel, over one or
    more rocprofv3 --pmc counter_collection.csv files (one counter set each)."""
    import csv
    import collections

    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = _kernel_short_name(r["Kernel_Name"])
                if name.startswith("zs::"):
                    vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: {"mean": statistics.fmean(v), "dispatches": len(v)} for c, v in sorted(cs.items())}
            for k, cs in sorted(vals.items())}


# The GIE page's own timings of its fused Triton kernels (fp32, torch.compile
# inference, 4096-atom diamond frame of the DPA4-Neo model, C = 32) on an
# NVIDIA RTX 5090 (GIE page, "Numbers" section).  Another GPU and real model
# inputs: reported beside the result for context, never as vs_baseline.
PAGES_FWD_US, PAGES_BWD_US = 200.0, 500.0


def pages_context(fb_us: float, nb: dict) -> dict:
    pages_us = PAGES_FWD_US + PAGES_BWD_US
    return {
        "hardware": "NVIDIA RTX 5090",
        "fwd_us": PAGES_FWD_US,
        "bwd_us": PAGES_BWD_US,
        "fwd_bwd_us": pages_us,
        "algorithmic_gbs": round((nb["fwd"] + nb["bwd"]) / (pages_us * 1e-6) / 1e9, 1),
        "time_ratio": round(pages_us / fb_us, 2),
        "note": "the pages' fused kernels on another GPU with real model inputs; context only",
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, w, budget_s: float = 12.0) -> dict:
    """The oracle (plain sequential C, one thread) on the same inputs: forward
    and backward timed separately, median over the passes that fit the budget
    (at most 40, about 12 s of CPU work on the headline frame)."""
    import oracle
    nbytes = algorithmic_bytes(w.n_edges, w.n_nodes, w.channels)
    fwd, bwd = [], []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.forward(x["coupling"], x["radial"], x["dst"], w.n_nodes)
        t1 = time.perf_counter()
        oracle.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"])
        t2 = time.perf_counter()
        fwd.append(t1 - t0)
        bwd.append(t2 - t1)
        if time.perf_counter() - t_start > budget_s or len(fwd) >= 40:
            break
    f_med, b_med = statistics.median(fwd), statistics.median(bwd)
    rec = {
        "value": round((nbytes["fwd"] + nbytes["bwd"]) / (f_med + b_med) / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{len(fwd)} full passes (forward + backward) of the {w.name} workload, "
                   f"medians {f_med * 1e3:.1f} ms forward + {b_med * 1e3:.1f} ms backward, "
                   f"single thread of {os.cpu_count()} visible"),
        "fwd_ms": round(f_med * 1e3, 2),
        "bwd_ms": round(b_med * 1e3, 2),
        "cpu_model": _cpu_model(),
        "cores_visible": os.cpu_count(),
    }
    rec["all_cores"] = cpu_baseline_all_cores(x, w, nbytes)
    return rec


def cpu_baseline_all_cores(x, w, nbytes, budget_s: float = 4.0) -> dict:
    """The oracle's K-thread variant (node-blocked forward keeping each node's
    edge order, edge-blocked backward; bitwise equal to the oracle) on every
    visible core, on the same inputs; the CSR it walks is the oracle's, built
    once outside the timing.  A separate figure: ``value`` above stays the
    single-thread oracle."""
    try:
        import oracle
        mt = oracle.get_mt()
        threads = os.cpu_count() or 1
        csr = oracle.csr(x["dst"], w.n_nodes)
        fwd, bwd = [], []
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            mt.forward(x["coupling"], x["radial"], x["dst"], w.n_nodes, threads, csr=csr)
            t1 = time.perf_counter()
            mt.backward(x["grad_out"], x["coupling"], x["radial"], x["dst"], threads)
            t2 = time.perf_counter()
            fwd.append(t1 - t0)
            bwd.append(t2 - t1)
            if time.perf_counter() - t_start > budget_s or len(fwd) >= 40:
                break
        f_med, b_med = statistics.median(fwd), statistics.median(bwd)
        return {
            "value": round((nbytes["fwd"] + nbytes["bwd"]) / (f_med + b_med) / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle, K-thread variant (bitwise equal)",
            "sample": (f"{len(fwd)} full passes of the {w.name} workload, medians "
                       f"{f_med * 1e3:.2f} ms forward + {b_med * 1e3:.2f} ms backward"),
            "fwd_ms": round(f_med * 1e3, 3),
            "bwd_ms": round(b_med * 1e3, 3),
        }
    except Exception as exc:   # the K-thread build needs gcc's OpenMP runtime
        return {"error": f"{type(exc).__name__}: {exc}"}


FLUSH_BYTES = 512 * 1024 * 1024   # above the 256 MB memory-side cache plus the L2s


class Flusher:
    """Evicts the frame from the caches before a cold sample.

    ``read``: a sum over a 512 MiB buffer written once up front, so the caches
    end up holding clean, unrelated lines and the sample pays for no
    write-back.  ``fill``: the buffer is overwritten instead, which leaves
    dirty lines whose write-back can fall inside the sample (kept as a second
    figure for comparison)."""

    def __init__(self, torch, dev):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.acc = torch.empty((), dtype=torch.float32, device=dev)
        self.torch = torch
        self.i = 0

    def __call__(self, mode: str) -> None:
        if mode == "read":
            self.torch.sum(self.buf, dim=0, out=self.acc)
        elif mode == "fill":
            self.i += 1
            self.buf.fill_(float(self.i))
        else:
            raise ValueError(mode)


FLUSH_NOTES = {"read": "512 MiB buffer read (summed) before each sample",
               "fill": "512 MiB buffer overwritten before each sample"}


def time_flushed(zs, torch, flusher, mode, cpl, rad, g, csr, out, gc, gr, nb,
                 steps: int) -> dict:
    """Forward + backward with the caches flushed first (``Flusher``), then
    forward and backward between two events; median over the samples."""
    ms = []
    for _ in range(steps + 2):
        flusher(mode)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        zs.zs_forward(cpl, rad, csr, out=out)
        zs.zs_backward(g, cpl, rad, csr, grad_coupling=gc, grad_radial=gr)
        b.record()
        ms.append((a, b))
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) * 1e3 for a, b in ms[2:]]
    med = statistics.median(t)
    gbs = (nb["fwd"] + nb["bwd"]) / (med * 1e-6) / 1e9
    return {"fwd_bwd_us_median": round(med, 2), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "samples": len(t),
            "note": FLUSH_NOTES[mode]}


def time_normalized(zs, torch, cpl, rad, x, csr, dev, steps: int) -> dict:
    """The same frame through the fused degree normalisation
    (zs_forward_normalized + zs_backward_normalized, CSR reused), timed with
    per-call events like the main steps, after the main timed region."""
    E, N, C = rad.shape[0], csr.n_nodes, rad.shape[2]
    cpl, rad = cpl.contiguous(), rad.contiguous()
    env = torch.from_numpy(x["env"]).to(dev)
    gy = torch.from_numpy(x["grad_out"]).to(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(-3, steps):
        if i >= 0:
            evs[i][0].record()
        y, out, norm = zs.zs_forward_normalized(cpl, rad, env, csr)
        if i >= 0:
            evs[i][1].record()
        zs.zs_backward_normalized(gy, out, norm, cpl, rad, csr)
        if i >= 0:
            evs[i][2].record()
    torch.cuda.synchronize()
    fwd_us = statistics.fmean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    bwd_us = statistics.fmean(e[1].elapsed_time(e[2]) for e in evs) * 1e3
    nb = algorithmic_bytes_normalized(E, N, C)
    gbs = (nb["fwd"] + nb["bwd"]) / ((fwd_us + bwd_us) * 1e-6) / 1e9
    return {"fwd_us": round(fwd_us, 2), "bwd_us": round(bwd_us, 2),
            "fwd_bwd_us": round(fwd_us + bwd_us, 2), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": nb,
            "note": "bwd_us covers the scatter backward and the two degree-gradient kernels"}


def copy_probe(torch, dev, reps: int = 10) -> dict:
    """A plain 256 MiB device-to-device copy (torch's copy kernel), median of
    ``reps`` event-timed copies: the bandwidth a streaming read + write reaches
    on this GPU in the same run."""
    n = COPY_CALIBRATION_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    us = statistics.median(a.elapsed_time(b) for a, b in evs) * 1e3
    moved = 2 * COPY_CALIBRATION_BYTES
    return {"gbs": round(moved / (us * 1e-6) / 1e9, 1), "bytes_moved": moved, "us": round(us, 2),
            "note": "torch device copy of 256 MiB (read + write), median of 10"}


# the other frames, and the headline shape with i.i.d. uniform destinations
# (Poisson degrees) as a secondary row of the headline
WORKLOADS_REPORTED = ("n1000", "skewed", "large", "headline_uniform")


def progress(msg: str) -> None:
    """A progress line on stderr (the JSON result is the only stdout line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_workloads(zs, torch, dev, names, steps: int) -> dict:
    """Warm and cache-flushed forward + backward of other frames, in this
    process after the headline's timed region.  Every pass is a step shaped
    like the headline's: CSR build, forward, backward, with an event around
    the forward and the backward (the build is not timed); per frame a few
    warmup passes, then ``steps`` back-to-back passes (warm) and
    ``min(steps, 20)`` passes each preceded by the read flush (flushed).
    Inputs are freed before the next frame."""
    rep = {}
    for name in names:
        w = synthetic.WORKLOADS[name]
        x = synthetic.make_inputs(w)
        E, N, C = w.n_edges, w.n_nodes, w.channels
        t = {k: torch.from_numpy(x[k]).to(dev) for k in ("dst", "coupling", "radial", "grad_out")}
        del x
        csr = zs.zs_build_csr(t["dst"], N)
        ws = torch.empty(max(zs.zs_csr_workspace_bytes(E, N), 1), dtype=torch.uint8, device=dev)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
        out = torch.empty((N, 16, C), device=dev)
        gc = torch.empty((E, 15), device=dev)
        gr = torch.empty((E, 3, C), device=dev)
        flusher = Flusher(torch, dev)
        nb = algorithmic_bytes(E, N, C)

        def pair(evs):
            zs.zs_build_csr(t["dst"], N, workspace=ws, out=csr, bad_flag=flag)
            evs[0].record()
            zs.zs_forward(t["coupling"], t["radial"], csr, out=out)
            evs[1].record()
            zs.zs_backward(t["grad_out"], t["coupling"], t["radial"], csr, grad_coupling=gc,
                           grad_radial=gr)
            evs[2].record()

        res = {}
        for mode, n in (("warm", steps), ("flushed", min(steps, 20))):
            for _ in range(3):
                pair([torch.cuda.Event(enable_timing=True) for _ in range(3)])
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
            for e in evs:
                if mode == "flushed":
                    flusher("read")
                pair(e)
            torch.cuda.synchronize()
            if int(flag.item()) != 0:
                raise RuntimeError(f"destination index out of range in workload {name}")
            fwd = statistics.median(e[0].elapsed_time(e[1]) for e in evs) * 1e3
            bwd = statistics.median(e[1].elapsed_time(e[2]) for e in evs) * 1e3
            fb = statistics.median(e[0].elapsed_time(e[2]) for e in evs) * 1e3
            gbs = (nb["fwd"] + nb["bwd"]) / (fb * 1e-6) / 1e9
            res[mode] = {"fwd_us": round(fwd, 2), "bwd_us": round(bwd, 2),
                         "fwd_bwd_us": round(fb, 2), "gbs": round(gbs, 1),
                         "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        rep[name] = {"n_nodes": N, "n_edges": E, "channels": C,
                     "algorithmic_bytes": nb["fwd"] + nb["bwd"],
                     "target_us_at_60pct": round((nb["fwd"] + nb["bwd"]) /
                                                 (0.6 * PEAK_HBM_GBS * 1e9) * 1e6, 1),
                     **res}
        del t, csr, ws, flag, out, gc, gr, flusher
        torch.cuda.empty_cache()
        progress(f"workload {name}: warm {res['warm']['fwd_bwd_us']} us, "
                 f"flushed {res['flushed']['fwd_bwd_us']} us")
    rep["note"] = ("steps of CSR build, forward, backward; medians per call of the forward and "
                   "the backward, with an event between them; flushed: " + FLUSH_NOTES["read"])
    return rep


PROTOCOL_WARMUP, PROTOCOL_SAMPLES = 12, 50


PROTOCOL_MODES = {"flushed": "read", "flushed_fill": "fill", "warm": None}


def protocol_child(zs, torch, dev, dst, cpl, rad, g, csr, ws, flag, out, gc, gr, N) -> dict:
    """One fresh process's share of the protocol: warmup, then samples of
    build / forward / backward with an event around each call, with the caches
    flushed before each sample (read flush, then fill flush) and without."""
    flusher = Flusher(torch, dev)

    def sample(evs):
        if evs:
            evs[0].record()
        zs.zs_build_csr(dst, N, workspace=ws, out=csr, bad_flag=flag)
        if evs:
            evs[1].record()
        zs.zs_forward(cpl, rad, csr, out=out)
        if evs:
            evs[2].record()
        zs.zs_backward(g, cpl, rad, csr, grad_coupling=gc, grad_radial=gr)
        if evs:
            evs[3].record()

    res = {}
    for mode, flush in PROTOCOL_MODES.items():
        for _ in range(PROTOCOL_WARMUP):
            sample(None)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
               for _ in range(PROTOCOL_SAMPLES)]
        for i in range(PROTOCOL_SAMPLES):
            if flush is not None:
                flusher(flush)
            sample(evs[i])
        torch.cuda.synchronize()
        if int(flag.item()) != 0:
            raise RuntimeError("destination index out of range in the synthetic input")

        def med(a, b):
            return statistics.median(e[a].elapsed_time(e[b]) for e in evs) * 1e3

        res[mode] = {"build_us": med(0, 1), "fwd_us": med(1, 2), "bwd_us": med(2, 3),
                     "fwd_bwd_us": med(1, 3)}
    return res


def run_protocol(args, nb) -> dict:
    """Runs the child processes (before this process initialises the GPU) and
    takes the median of their medians."""
    cmd = [sys.executable, os.path.abspath(__file__), "--protocol-child",
           "--workload", args.workload, "--inputs", args.inputs]
    if args.channels is not None:
        cmd += ["--channels", str(args.channels)]
    per = []
    for _ in range(args.processes):
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if r.returncode != 0:
            raise RuntimeError(f"protocol child failed ({r.returncode}): {r.stderr[-2000:]}")
        per.append(json.loads(r.stdout.strip().splitlines()[-1]))
        progress(f"protocol child {len(per)}/{args.processes}: flushed "
                 f"{per[-1]['flushed']['fwd_bwd_us']:.1f} us, warm {per[-1]['warm']['fwd_bwd_us']:.1f} us")
    rep = {"processes": args.processes, "warmup": PROTOCOL_WARMUP, "samples": PROTOCOL_SAMPLES}
    for mode in PROTOCOL_MODES:
        agg = {k: round(statistics.median(p[mode][k] for p in per), 2) for k in per[0][mode]}
        gbs = (nb["fwd"] + nb["bwd"]) / (agg["fwd_bwd_us"] * 1e-6) / 1e9
        agg["gbs"] = round(gbs, 1)
        agg["hbm_frac"] = round(gbs / PEAK_HBM_GBS, 4)
        rep[mode] = agg
    rep["per_process_fwd_bwd_us"] = {m: [round(p[m]["fwd_bwd_us"], 2) for p in per]
                                     for m in PROTOCOL_MODES}
    rep["note"] = ("median over processes of each process's median; the fwd+bwd span has an "
                   "event between the two calls; flushed: " + FLUSH_NOTES["read"] +
                   "; flushed_fill: " + FLUSH_NOTES["fill"])
    return rep


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="headline", choices=sorted(synthetic.WORKLOADS))
    ap.add_argument("--channels", type=int, default=None,
                    help="run the workload's frame (same N, E, destinations and seed) with this "
                         "channel count instead of its own")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-flushed and normalised timings (so that counter runs "
                         "see only the plain path's launches)")
    ap.add_argument("--inputs", default="contiguous", choices=["contiguous", "views"],
                    help="views: coupling read in place from a packed (E, 46) Wigner band and "
                         "radial features sliced from an (E, 5, C) tensor (strided entry points)")
    ap.add_argument("--write-traffic", nargs="+", metavar="CSV",
                    help="FETCH_CSV WRITE_CSV [OUT_JSON]: summarize two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) into "
                         "profiles/traffic_headline.json (or OUT_JSON) and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print the mean per dispatch of every counter in these rocprofv3 --pmc "
                         "counter_collection.csv files, per zs:: kernel, and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 256 MiB device copy three times "
                         "(reference kernel for scaling rocprofv3 byte counters)")
    ap.add_argument("--flush", choices=["none", "read", "fill"], default="none",
                    help="empty the caches before every warmup and timed step (read: sum a "
                         "512 MiB buffer; fill: overwrite it), e.g. for counter runs of cold "
                         "launches; the line's value is then the cold figure")
    ap.add_argument("--processes", type=int, default=3,
                    help="fresh-process protocol in this many child processes (0: skip it)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the warm and cache-flushed timings of the other frames "
                         "(1000-node, skewed, 16384-node) that the headline run reports")
    ap.add_argument("--protocol-child", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.write_traffic:
        if len(args.write_traffic) not in (2, 3):
            ap.error("--write-traffic takes FETCH_CSV WRITE_CSV [OUT_JSON]")
        print(json.dumps(write_traffic(*args.write_traffic), indent=1))
        return 0
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by destination node with no exchange, see the design notes)",
              file=sys.stderr)
        return 2

    w = synthetic.WORKLOADS[args.workload]
    if args.channels is not None and args.channels != w.channels:
        w = synthetic.custom(f"{w.name}_c{args.channels}", w.n_nodes, w.n_edges, args.channels,
                             w.seed, w.dst_kind, w.envelope)
    # the child processes run before this process initialises the GPU
    protocol = (run_protocol(args, algorithmic_bytes(w.n_edges, w.n_nodes, w.channels))
                if args.processes > 0 and not args.protocol_child else None)

    import torch
    import edge_node_scatter_amd as zs

    x = synthetic.make_inputs(w)
    dev = torch.device("cuda:0")
    zs.load()
    dst = torch.from_numpy(x["dst"]).to(dev)
    E, N, C = w.n_edges, w.n_nodes, w.channels
    if args.inputs == "views":
        band = torch.zeros((E, 3 * 16 - 2), device=dev)
        cpl = zs.coupling_from_band(band)
        cpl.copy_(torch.from_numpy(x["coupling"]).to(dev))
        wide = torch.zeros((E, 5, C), device=dev)
        rad = wide[:, 1:4]
        rad.copy_(torch.from_numpy(x["radial"]).to(dev))
    else:
        cpl = torch.from_numpy(x["coupling"]).to(dev)
        rad = torch.from_numpy(x["radial"]).to(dev)
    g = torch.from_numpy(x["grad_out"]).to(dev)
    csr = zs.Csr(torch.empty(N + 1, dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev),
                 torch.empty(E, dtype=torch.int32, device=dev), N,
                 torch.empty(N, dtype=torch.int32, device=dev))
    ws = torch.empty(max(zs.zs_csr_workspace_bytes(E, N), 1), dtype=torch.uint8, device=dev)
    flag = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.empty((N, 16, C), device=dev)
    gc = torch.empty((E, 15), device=dev)
    gr = torch.empty((E, 3, C), device=dev)

    step_flusher = Flusher(torch, dev) if args.flush != "none" else None

    def step(evs=None, split=False):
        """One step.  evs: [before build, before forward, between (split only),
        after backward]; the forward + backward time is the span of one event
        pair (an event between the two calls adds a few microseconds of its own)."""
        if step_flusher is not None:
            step_flusher(args.flush)
        if evs is not None:
            evs[0].record()
        zs.zs_build_csr(dst, N, workspace=ws, out=csr, bad_flag=flag)
        if evs is not None:
            evs[1].record()
        zs.zs_forward(cpl, rad, csr, out=out)
        if evs is not None and split:
            evs[2].record()
        zs.zs_backward(g, cpl, rad, csr, grad_coupling=gc, grad_radial=gr)
        if evs is not None:
            evs[3].record()

    if args.protocol_child:
        print(json.dumps(protocol_child(zs, torch, dev, dst, cpl, rad, g, csr, ws, flag, out, gc,
                                        gr, N)), flush=True)
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(flag.item()) != 0:
        raise RuntimeError("destination index out of range in the synthetic input")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    progress(f"timed steps done: {args.steps} steps in {wall:.3f} s")
    if int(flag.item()) != 0:
        raise RuntimeError("destination index out of range in the synthetic input")

    build_ms = [ev[0].elapsed_time(ev[1]) for ev in events]
    fb_ms = [ev[1].elapsed_time(ev[3]) for ev in events]
    # per-call split (for the per-kernel figures and the roofline): the same steps
    # again with an event between forward and backward
    split_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                    for _ in range(args.steps)]
    for i in range(args.steps):
        step(split_events[i], split=True)
    torch.cuda.synchronize()
    fwd_ms = [ev[1].elapsed_time(ev[2]) for ev in split_events]
    bwd_ms = [ev[2].elapsed_time(ev[3]) for ev in split_events]
    mean = statistics.fmean
    nb = algorithmic_bytes(E, N, C)
    fwd_us, bwd_us, build_us = mean(fwd_ms) * 1e3, mean(bwd_ms) * 1e3, mean(build_ms) * 1e3
    fb_us = mean(fb_ms) * 1e3
    gbs = (nb["fwd"] + nb["bwd"]) / (fb_us * 1e-6) / 1e9
    bwd_gbs = nb["bwd"] / (bwd_us * 1e-6) / 1e9
    # the committed counter summary covers the headline frame with contiguous inputs only
    headline_frame = w.name == "headline" and args.inputs == "contiguous"
    traffic = load_traffic("zs_bwd_staged_kernel") if headline_frame else None

    rec = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: N={N} nodes, E={E} edges, C={C} channels, lmax=3, fp32",
            "n_nodes": N, "n_edges": E, "channels": C, "dst": w.dst_kind,
            "inputs": args.inputs, "flush_before_step": args.flush,
        },
        "fwd_bwd_us": round(fb_us, 2),
        "fwd_us": round(fwd_us, 2),
        "bwd_us": round(bwd_us, 2),
        "build_us": round(build_us, 2),
        "fwd_bwd_us_median": round(statistics.median(fb_ms) * 1e3, 2),
        "edges_per_s": round(E / (fb_us * 1e-6), 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "algorithmic_bytes": nb,
        "roofline": {
            "kernel": "zs_bwd_staged_kernel",
            "bound": "hbm",
            "achieved": round(bwd_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(bwd_gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nb["bwd"],
            "avg_launch_us": round(bwd_us, 2),
        },
        "kernels": {
            k: kernel_roofline(k, nb[part], us, headline_frame)
            for k, part, us in (("zs_fwd_staged_kernel", "fwd", fwd_us),
                                ("zs_bwd_staged_kernel", "bwd", bwd_us))
        },
        "source_hash": {fam: kernel_source_hash(fam) for fam in KERNEL_SOURCES},
        "input_hashes": synthetic.fingerprint(x),
    }
    if w.name == "headline" and args.inputs == "contiguous":
        rec["pages_context"] = pages_context(fb_us, nb)
    if not args.no_extras:
        flusher = Flusher(torch, dev)
        n_flushed = min(args.steps, 20)
        rec["flushed"] = time_flushed(zs, torch, flusher, "read", cpl, rad, g, csr, out, gc, gr,
                                      nb, n_flushed)
        rec["flushed_fill"] = time_flushed(zs, torch, flusher, "fill", cpl, rad, g, csr, out, gc,
                                           gr, nb, n_flushed)
        del flusher
        rec["normalized"] = time_normalized(zs, torch, cpl, rad, x, csr, dev, args.steps)
        rec["copy_probe"] = copy_probe(torch, dev)
    if protocol is not None:
        rec["protocol"] = protocol
    if (w.name == "headline" and args.inputs == "contiguous" and args.channels is None
            and not args.no_workloads and not args.no_extras):
        del out, gc, gr, ws
        rec["workloads"] = time_workloads(zs, torch, dev, WORKLOADS_REPORTED, args.steps)
    if args.calibrate_copy:
        src = torch.empty(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst_copy = torch.empty_like(src)
        for _ in range(3):
            dst_copy.copy_(src)
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = COPY_CALIBRATION_BYTES
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
