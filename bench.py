"""Benchmark of the OSDN forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--backward]

One step = one full forward (osdn_forward: phase 1 preconditioner scan and
phase 2 chunked WY delta rule) over the workload's synthetic batch, inputs
resident in HBM, outputs and workspace preallocated. Other workloads time
gdn2_forward, osdn_gated_forward or one recurrent decode call the same way.
With --backward a step is the backward of the workload's forward instead
(osdn_backward, osdn_gated_backward or gdn2_backward: every input's gradient
from seeded output adjoints).

Prints one JSON line: throughput (tokens/s = B*T per step time), the HBM
roofline of the whole step (algorithmic bytes of the forward per its step
time), the dominant kernel beside it, per-kernel durations measured live by
the library's HIP-event timing on the launch stream, and the fp64 CPU oracle
timed on the host cores (before the GPU is touched).
"""
import argparse
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
HOST_CPU_SHARE = 16            # host threads a one-GPU job may use

_CSRC = os.path.join(ROOT, "delta_rule_recurrent_scan_amd", "csrc")
_KERNEL_SOURCES = {
    "precond_prep": ["precond_scan.hip"],
    "precond_chain": ["precond_scan.hip"],
    "precond_ktilde": ["precond_scan.hip"],
    "precond_rho": ["precond_scan.hip"],
    "wy_prep": ["wy_chunk.hip"],
    "wy_prep_fused": ["wy_chunk.hip"],
    "wy_scan": ["wy_chunk.hip"],
    "gdn2_prep": ["wy_chunk.hip"],
    "gdn2_scan": ["wy_chunk.hip"],
    "gated_prep": ["wy_chunk.hip"],
    "gated_prep_fused": ["wy_chunk.hip"],
    "gated_scan": ["wy_chunk.hip"],
    "osdn_decode": ["decode.hip"],
    "gdn2_decode": ["decode.hip"],
    "osdn_bwd_record": ["backward.hip", "bwd_common.hpp", "row_state.hpp"],
    "osdn_bwd": ["backward.hip", "bwd_common.hpp", "row_state.hpp"],
    "osdn_bwd_learner": ["backward.hip", "bwd_common.hpp", "row_state.hpp"],
    "gated_bwd_record": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
    "gated_bwd": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
    "gated_bwd_learner": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
    "gdn2_bwd_record": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
    "gdn2_bwd": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
    "gdn2_bwd_out": ["backward_gated.hip", "bwd_common.hpp", "row_state.hpp"],
}
PRECOND_CHUNK = 64  # phase-1 chunk length (fixed in the library)


def source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES.get(kernel, []) + ["device_common.hpp"]:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, run):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by the copy-kernel calibration) of this run
    (the workload name, with "-backward" for the backward), or None when
    there are none or the kernel's sources have changed since."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))["runs"][run][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel):
        return None
    return rec["bytes"]


# ---------------------------------------------------------------------------
# Algorithmic work: the bytes and flops the method itself must move and do
# ---------------------------------------------------------------------------

def _s(w):
    return 2 if w.dtype == "bf16" else 4


def path_bytes(w):
    """Algorithmic HBM bytes of one call over the whole workload: what the
    method itself must read and write once. Per token-head: OSDN q, k (Dk
    each) and v (Dv) read, o (Dv) written, beta and r read; GDN-2 q, k, b
    (Dk), v, w (Dv), log alpha (Dk fp32), o; gated OSDN adds log alpha to
    OSDN. Per (batch, head) stream: the fp32 final state written, and for
    OSDN d0 read and d_T written (Dk fp32 each). Decode: the state read and
    written once plus the call's tokens."""
    s, dk, dv = _s(w), w.Dk, w.Dv
    th, bh = w.B * w.H * w.T, w.B * w.H
    gates = 4 + (4 if w.apf else 0)
    if w.state:
        return bh * decode_bytes_per_head(w)
    if w.kind == "gdn2":
        tok = (3 * dk + 2 * dv) * s + 4 * dk + dv * s
        return th * tok + bh * dk * dv * 4
    tok = (2 * dk + dv) * s + dv * s + gates + (4 * dk if w.decay else 0)
    return th * tok + bh * (dk * dv * 4 + 2 * dk * 4)


def backward_bytes(w):
    """Algorithmic HBM bytes of one backward call: every forward input read
    once (path_bytes' token inputs, without o), the output adjoint do read
    (Dv, dtype), every gradient written once in fp32 (per token-head: OSDN
    q, k, v, beta, r; gated OSDN adds log alpha; GDN-2 q, k, v, log alpha,
    b, w), and per stream the state's adjoint read and S0's gradient written
    (fp32), with OSDN's d adjoints and eta's gradient."""
    s, dk, dv = _s(w), w.Dk, w.Dv
    th, bh = w.B * w.H * w.T, w.B * w.H
    if w.kind == "gdn2":
        tok_in = (3 * dk + 2 * dv) * s + 4 * dk + dv * s
        tok_out = (4 * dk + 2 * dv) * 4
        return th * (tok_in + tok_out) + bh * 2 * dk * dv * 4
    gates = 4 + (4 if w.apf else 0)
    tok_in = (2 * dk + dv) * s + gates + (4 * dk if w.decay else 0) + dv * s
    tok_out = (2 * dk + dv + 2) * 4 + (4 * dk if w.decay else 0)
    return th * (tok_in + tok_out) + bh * (2 * dk * dv * 4 + 2 * dk * 4 + 4)


def decode_bytes_per_head(w):
    """Algorithmic bytes per (batch, head) of one decode call: the fp32 state
    read and written once, plus the call's tokens (inputs and outputs) and,
    for OSDN, the preconditioner read and written."""
    s = _s(w)
    state = 2 * w.Dk * w.Dv * 4
    if w.kind == "osdn":
        tok = (2 * w.Dk + w.Dv) * s + w.Dv * s + 4 + (4 if w.apf else 0)
        return state + 2 * w.Dk * 4 + w.T * tok
    tok = (3 * w.Dk + 2 * w.Dv) * s + 4 * w.Dk + w.Dv * s
    return state + w.T * tok


def kernel_bytes_per_token_head(w):
    """Interface bytes per token-head of each kernel: everything it reads
    and writes once, the workspace arrays handed between kernels included
    (a per-kernel figure beside the path's own algorithmic bytes)."""
    s = _s(w)
    dk, dv, C, C1 = w.Dk, w.Dv, w.chunk, PRECOND_CHUNK
    gates = 4 + (4 if w.apf else 0)
    rec = (3 * C1 + 8 + C1 * C1) * 4.0 / C1   # phase-1 chunk record
    dent = dk * 4.0 / C1                       # d at each chunk entry
    frags = (2 * dk + dv + C) * s
    frags_g = frags + dk * s + 4.0 * dk / C
    return {
        "precond_prep": dk * s + gates + rec,
        "precond_chain": dk * s + rec + 4 + dent,
        "precond_ktilde": 2 * dk * s + 4 * (C1 + 4.0) / C1 + 4 + dent,
        "wy_prep": (3 * dk + dv) * s + 4 + frags,
        "wy_prep_fused": (2 * dk + dv) * s + 4 + 4 * (C1 + 4.0) / C1 + 4 + dent
        + frags,
        "wy_scan": frags + dk * s + dv * s,
        "gdn2_prep": (3 * dk + 2 * dv) * s + 4 * dk + frags_g,
        "gdn2_scan": frags_g + dv * s,
        "gated_prep": (3 * dk + dv) * s + 4 + 4 * dk + frags_g,
        "gated_scan": frags_g + dv * s,
        "gated_prep_fused": (2 * dk + dv) * s + 4 + 4 * dk
        + 4 * (C1 + 4.0) / C1 + 4 + dent + frags_g,
    }


def flops_per_token_head(w):
    """Chunk-form flops per token-head of phase 2: state chain 4 Dk Dv,
    inter-chunk output 2 Dk Dv, intra-chunk Gram, W and scores
    2 C (3 Dk + 2 Dv), triangular inverse about C^2 / 3."""
    C, dk, dv = w.chunk, w.Dk, w.Dv
    return 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3.0


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores (runs before the GPU is
# touched, so that worker processes fork from a process with no GPU state)
# ---------------------------------------------------------------------------

_UNITS = {}


def _oracle_unit(i):
    """Run the oracle on unit i of the workload (a (batch, head) stream of a
    forward; a batch row of all heads of a decode call); returns seconds."""
    from oracle import recurrence as R
    w, arrs = _UNITS["w"], _UNITS["arrs"]
    if w.state:
        sl = (slice(i, i + 1), slice(None))
    else:
        b, h = divmod(i, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
    a = {k: (None if v is None else v[sl]) for k, v in arrs.items()}
    t0 = time.perf_counter()
    if _UNITS.get("backward"):
        from oracle import backward as BW
        if w.kind == "gdn2":
            BW.gdn2_backward_ref(a["q"], a["k"], a["v"], a["log_alpha"],
                                 a["b"], a["w"], a.get("S0"), a["do"],
                                 a.get("dS_T"))
        elif w.decay:
            BW.osdn_gated_backward_ref(a["q"], a["k"], a["v"], a["beta"],
                                       a["log_alpha"], a["r"], w.eta,
                                       a.get("d0"), a.get("S0"), a["do"],
                                       a.get("dS_T"), a.get("dd_T"))
        else:
            BW.osdn_backward_ref(a["q"], a["k"], a["v"], a["beta"], a["r"],
                                 w.eta, a.get("d0"), a.get("S0"), a["do"],
                                 a.get("dS_T"), a.get("dd_T"))
    elif w.kind == "gdn2":
        R.gdn2_ref(a["q"], a["k"], a["v"], a["log_alpha"], a["b"], a["w"],
                   a.get("S0"))
    elif w.decay:
        R.osdn_gated_ref(a["q"], a["k"], a["v"], a["beta"], a["log_alpha"],
                         a["r"], w.eta, a.get("d0"), a.get("S0"))
    else:
        R.osdn_ref(a["q"], a["k"], a["v"], a["beta"], a["r"], w.eta,
                   a.get("d0"), a.get("S0"))
    return time.perf_counter() - t0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s=10.0, cot=None):
    """The fp64 NumPy oracle as it stands, on a bounded sample of the
    workload: (1) one thread, whole units in turn until budget_s is spent;
    (2) a fork pool of min(16, cpu_count) processes (started before the
    timed region) over 2 units each (decode: every unit, one slice per
    process). Both scale the sample to the whole workload (units are
    independent).
    `value` is the pool figure; `cores` the processes it used."""
    keys = ("q", "k", "v", "beta", "r", "log_alpha", "b", "w", "S0", "d0")
    _UNITS["w"] = w
    _UNITS["backward"] = cot is not None
    _UNITS["arrs"] = {k: W.to_f64(inp[k]) for k in keys
                      if isinstance(inp.get(k), torch.Tensor)}
    if cot is not None:
        keys += ("do", "dS_T", "dd_T")
        _UNITS["arrs"].update({k: W.to_f64(v) for k, v in cot.items()
                               if isinstance(v, torch.Tensor)})
    for k in keys:
        _UNITS["arrs"].setdefault(k, None)
    n_units = w.B if w.state else w.B * w.H
    unit = "batch row (all heads)" if w.state else "(batch, head) stream"
    t_used, done = 0.0, 0
    while done < n_units and t_used < budget_s:
        t_used += _oracle_unit(done)
        done += 1
    single = w.B * w.T / (t_used / done * n_units)
    procs = max(1, min(HOST_CPU_SHARE, os.cpu_count() or 1))
    # forward units take seconds: two per process; decode units take about a
    # millisecond: all of them, in one slice per process
    n_pool = n_units if w.state else min(n_units, 2 * procs)
    chunk = max(1, n_pool // procs) if w.state else 1
    ctx = mp.get_context("fork")
    with ctx.Pool(procs) as pool:
        pool.map(abs, range(procs))           # processes started and idle
        t0 = time.perf_counter()
        pool.map(_oracle_unit, range(n_pool), chunksize=chunk)
        wall = time.perf_counter() - t0
    pooled = w.B * w.T / (wall * n_units / n_pool)
    return {"value": pooled, "unit": "tokens/s", "cores": procs,
            "kind": "oracle",
            "sample": ("fp64 NumPy adjoint of the token recurrence"
                       if cot is not None else
                       "fp64 NumPy token recurrence")
            + "; %d of %d units (one unit "
                      "= one %s at T=%d) on a fork pool of %d processes, "
                      "scaled to the whole workload" % (n_pool, n_units, unit,
                                                        w.T, procs),
            "cpu_model": _cpu_model(),
            "host_cpu_count": os.cpu_count(),
            "single_thread": {"value": single, "unit": "tokens/s",
                              "cores": 1,
                              "sample": "%d of %d units, one thread, "
                                        "%.1f s" % (done, n_units, t_used)}}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def _quantiles(ts):
    ts = sorted(ts)
    n = len(ts)
    return {"median_ms": ts[n // 2], "min_ms": ts[0],
            "p90_ms": ts[min(n - 1, int(np.ceil(0.9 * n)) - 1)]}


def timed_steps(step, args):
    """Warm up, then time exactly args.steps steps back to back (synchronised
    on both sides): the wall time per step. Then, outside that region: the
    same number of steps each bracketed by HIP events on the launch stream
    (median / min / p90), one more pass with the library's per-kernel event
    timing, and cold steps (each timed alone after 1 GiB has been written
    elsewhere, so that no input is left in the memory-side cache or L2)."""
    import delta_rule_recurrent_scan_amd as osdn
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per_step = _quantiles([a.elapsed_time(b) for a, b in ev])
    osdn.kernel_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    osdn.kernel_timing(False)
    rec = osdn.kernel_times()
    kt = {n: {"launches_per_step": cnt / args.steps, "mean_launch_ms": ms,
              "ms_per_step": ms * cnt / args.steps}
          for n, (cnt, ms) in rec.items()}
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    cold = []
    for i in range(args.steps):
        flush.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold_q = _quantiles(cold)
    cold_q["note"] = ("each step timed alone after writing 1 GiB elsewhere "
                      "(inputs not in the memory-side cache or L2)")
    return wall * 1e3 / args.steps, per_step, kt, cold_q


def roofline(w, ms_step, kt, backward=False):
    """HBM roofline of the whole step: the forward's algorithmic bytes (see
    path_bytes) over the measured step time, against the 8 TB/s peak.
    `traffic` is the HBM bytes all kernels of a step move (rocprofv3
    FETCH_SIZE / WRITE_SIZE, calibrated), null unless every kernel's
    counters match its current sources. The dominant (longest) kernel is
    reported beside it: its mean launch duration, its own interface bytes
    per launch over that duration, and the path's bytes over it."""
    alg = backward_bytes(w) if backward else path_bytes(w)
    achieved = alg / (ms_step * 1e-3) / 1e9
    run = w.name + ("-backward" if backward else "")
    traffic = 0.0
    for n, k in kt.items():
        b = measured_traffic(n, run)
        if b is None:
            traffic = None
            break
        traffic += b * k["launches_per_step"]
    dom = max(kt, key=lambda n: kt[n]["ms_per_step"])
    kd = kt[dom]
    kb = kernel_bytes_per_token_head(w).get(dom)
    th = w.B * w.H * w.T
    iface = None
    if kb is not None:
        iface = kb * th / kd["launches_per_step"]
    elif w.state:
        iface = alg / kd["launches_per_step"]
    dk = {"name": dom, "mean_launch_ms": kd["mean_launch_ms"],
          "launches_per_step": kd["launches_per_step"],
          "interface_bytes": iface,
          "interface_GBs": (None if iface is None
                            else iface / (kd["mean_launch_ms"] * 1e-3) / 1e9),
          "path_bytes_frac": alg / kd["launches_per_step"]
          / (kd["mean_launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
          "traffic": measured_traffic(dom, run)}
    return {"scope": "whole step", "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "traffic_ratio": None if traffic is None else traffic / alg,
            "alg_bytes": alg, "ms": ms_step, "dominant_kernel": dk}


# ---------------------------------------------------------------------------
# Steps
# ---------------------------------------------------------------------------

def make_step(w, x, dt, dev):
    import delta_rule_recurrent_scan_amd as osdn
    L = osdn.load_library()
    P = osdn._ptr
    code = {torch.float32: 0, torch.bfloat16: 1}[dt]
    sp = torch.cuda.current_stream(dev).cuda_stream
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    if w.state:
        S = x["S0"].clone()
        if w.kind == "osdn":
            d = x["d0"].clone()
            return lambda: osdn.osdn_decode(x["q"], x["k"], x["v"], x["beta"],
                                            S, d, r=x["r"], eta=x["eta"],
                                            out=o)
        return lambda: osdn.gdn2_decode(x["q"], x["k"], x["v"],
                                        x["log_alpha"], x["b"], x["w"], S,
                                        out=o)
    if w.kind == "gdn2":
        S_T = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32,
                          device=dev)
        ws_n = L.gdn2_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                              w.chunk, code)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

        def step():
            rc = L.gdn2_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code,
                                P(x["q"]), P(x["k"]), P(x["v"]),
                                P(x["log_alpha"]), P(x["b"]), P(x["w"]), None,
                                1.0, P(o), P(S_T), P(ws), ws.numel(), sp)
            if rc:
                raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))
        return step
    S_T = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    d_T = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    if w.decay:
        ws_n = L.osdn_gated_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                                    w.chunk, code)
        ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)
        return lambda: osdn.osdn_gated_forward(
            x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], x["r"],
            x["eta"], chunk=w.chunk, out=(o, S_T, d_T), workspace=ws)
    ws_n = L.osdn_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk,
                                          code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        rc = L.osdn_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code,
                            P(x["q"]), P(x["k"]), P(x["v"]), P(x["beta"]),
                            P(x["r"]), float(x["eta"]), None, None, 1.0, P(o),
                            P(S_T), P(d_T), None, None, P(ws), ws.numel(), sp)
        if rc:
            raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))
    return step


def make_backward_step(w, x, c, dev):
    """One backward call over the whole workload, gradients and workspace
    preallocated."""
    import delta_rule_recurrent_scan_amd as osdn
    f32 = torch.float32
    B, H, T, Dk, Dv = w.B, w.H, w.T, w.Dk, w.Dv
    e = lambda *shape: torch.empty(shape, dtype=f32, device=dev)
    if w.kind == "gdn2":
        g = dict(q=e(B, H, T, Dk), k=e(B, H, T, Dk), v=e(B, H, T, Dv),
                 log_alpha=e(B, H, T, Dk), b=e(B, H, T, Dk), w=e(B, H, T, Dv),
                 S0=e(B, H, Dk, Dv))
        n = osdn.gdn2_backward_workspace_bytes(B, H, T, Dk, Dv)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        return lambda: osdn.gdn2_backward(
            x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], c["do"],
            dS_T=c["dS_T"], out=g, workspace=ws)
    g = dict(q=e(B, H, T, Dk), k=e(B, H, T, Dk), v=e(B, H, T, Dv),
             beta=e(B, H, T), r=e(B, H, T), eta=e(B, H), d0=e(B, H, Dk),
             S0=e(B, H, Dv, Dk))
    if w.decay:
        g["log_alpha"] = e(B, H, T, Dk)
        n = osdn.gated_backward_workspace_bytes(B, H, T, Dk, Dv)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        return lambda: osdn.osdn_gated_backward(
            x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], c["do"],
            r=x["r"], eta=x["eta"], dS_T=c["dS_T"], dd_T=c["dd_T"], out=g,
            workspace=ws)
    n = osdn.backward_workspace_bytes(B, H, T, Dk, Dv)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    return lambda: osdn.osdn_backward(
        x["q"], x["k"], x["v"], x["beta"], c["do"], r=x["r"], eta=x["eta"],
        dS_T=c["dS_T"], dd_T=c["dd_T"], out=g, workspace=ws)


def metric_name(w, backward=False):
    if backward:
        label = ("GDN-2" if w.kind == "gdn2" else
                 "OSDN on a per-channel-decay backbone" if w.decay else "OSDN")
        return ("%s backward tokens/s + %% HBM roofline, H=16 d=128 T=4096, "
                "1 GPU" % label)
    if w.state:
        label = "OSDN" if w.kind == "osdn" else "GDN-2"
        return ("%s recurrent decode tokens/s + %% HBM roofline, B=%d H=%d "
                "d=%d, 1 GPU" % (label, w.B, w.H, w.Dk))
    if w.kind == "gdn2":
        return "GDN-2 forward tokens/s + % HBM roofline, H=16 d=128 T=4096, 1 GPU"
    if w.decay:
        return ("OSDN on a per-channel-decay backbone forward tokens/s + % "
                "HBM roofline, H=16 d=128 T=4096, 1 GPU")
    return "OSDN forward tokens/s + % HBM/MFMA roofline, H=16 d=128 T=4096, 1 GPU"


def calibrate_copy(args):
    n = 512 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    print(json.dumps({"calibration": "fp32 scale copy", "bytes_read": n * 4,
                      "bytes_written": n * 4, "ms": ms,
                      "GBs": 2 * n * 4 / (ms * 1e-3) / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="osdn-1.3b-apf",
                    choices=[w.name for w in W.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward of the workload's forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain fp32 scale-by-one kernel over 512 MiB "
                         "(reads and writes exactly 512 MiB each per step), "
                         "to scale hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(the forward shards over (batch, head) streams with no "
              "exchange between GPUs). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if torch.cuda.device_count() < 1:
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args)
        return

    w = W.BY_NAME[args.workload]
    if args.backward and w.state:
        print("--backward times a whole-sequence backward; pick a forward "
              "workload", file=sys.stderr)
        sys.exit(2)
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w) if args.backward else None
    cpu = (None if args.no_cpu_baseline
           else cpu_baseline(w, inp, cot=cot))

    import delta_rule_recurrent_scan_amd as osdn
    osdn.load_library()
    dev = torch.device("cuda:0")
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
         for k, v in inp.items()}
    dt = W.torch_dtype(w.dtype)
    if args.backward:
        c = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
             for k, v in cot.items()}
        step = make_backward_step(w, x, c, dev)
    else:
        step = make_step(w, x, dt, dev)
    ms_step, per_step, kt, cold = timed_steps(step, args)

    config = {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "Dk": w.Dk,
              "Dv": w.Dv}
    if not w.state:
        config["chunk"] = w.chunk
    if w.kind == "osdn":
        config.update(forgetting_gate=w.apf, eta=w.eta)
    rec = {
        "metric": metric_name(w, args.backward),
        "value": w.B * w.T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": config,
        "roofline": roofline(w, ms_step, kt, args.backward),
        "step_ms": per_step,
        "cold_step": cold,
        "kernels": kt,
    }
    if args.backward:
        config["pass"] = "backward"
        alg = backward_bytes(w)
        rec["roofline_cold"] = {
            "achieved": alg / (cold["median_ms"] * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": alg / (cold["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
    elif not w.state:
        flops = flops_per_token_head(w) * w.B * w.H * w.T
        rec["mfma"] = {"chunk_form_flops": flops,
                       "TFLOPs": flops / (ms_step * 1e-3) / 1e12,
                       "peak": MFMA_BF16_PEAK_TFLOPS,
                       "frac": flops / (ms_step * 1e-3) / 1e12
                       / MFMA_BF16_PEAK_TFLOPS}
    else:
        alg = path_bytes(w)
        rec["roofline_cold"] = {
            "achieved": alg / (cold["median_ms"] * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": alg / (cold["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
