"""Benchmark of the OSDN forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward (osdn_forward: phase 1 preconditioner scan and
phase 2 chunked WY delta rule; or gdn2_forward for --workload gdn2-1.3b) over
the workload's synthetic batch, inputs resident in HBM, outputs and
workspace preallocated. Per-kernel durations are measured live over the
timed region by the library's kernel timing, which records HIP events on the
launch stream around every kernel.

Prints one JSON line with the throughput (tokens/s = B*T per step time), the
roofline of the dominant kernel and the CPU-oracle baseline.
"""
import argparse
import json
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
}
PRECOND_CHUNK = 64  # phase-1 chunk length (fixed in the library)


def source_sha(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[kernel] + ["device_common.hpp", "launch.hpp"]:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by the copy-kernel calibration), or None when
    they were taken on another workload or on kernel sources that have
    changed since."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(kernel) or rec.get("workload") != workload:
        return None
    return rec["bytes"]


def path_bytes_per_token_head(w, apf):
    """Whole OSDN path: q, k (Dk each) and v (Dv) read, o (Dv) written,
    beta (and r) read."""
    s = 2 if w.dtype == "bf16" else 4
    return (2 * w.Dk + w.Dv) * s + w.Dv * s + 4 + (4 if apf else 0)


def kernel_bytes_per_token_head(w, apf=False):
    """Algorithmic bytes per token-head of each kernel: everything its
    interface reads and writes once (inputs, outputs and the workspace
    arrays handed from one kernel to the next)."""
    s = 2 if w.dtype == "bf16" else 4
    dk, dv, C, C1 = w.Dk, w.Dv, w.chunk, PRECOND_CHUNK
    gates = 4 + (4 if apf else 0)
    rec = (2 * C1 + 4 + C1 * C1) * 4.0 / C1   # phase-1 chunk record
    dent = dk * 4.0 / C1                       # d at each chunk entry
    # S0-independent chunk operands: Wk, X', U and the scores P; GDN-2 adds
    # its decayed queries and exit decays
    frags = (2 * dk + dv + C) * s
    frags_g = frags + dk * s + 4.0 * dk / C
    return {
        # k, beta, r -> record
        "precond_prep": dk * s + gates + rec,
        # k, record -> g, d entries
        "precond_chain": dk * s + rec + 4 + dent,
        # k, log gate prefix, g, d entries -> k~
        "precond_ktilde": 2 * dk * s + 4 * (C1 + 4.0) / C1 + 4 + dent,
        # q, k, k~, v, beta -> Wk, X', U, P
        "wy_prep": (3 * dk + dv) * s + 4 + frags,
        # q, k, v, beta, log gate prefix, g, d entries -> Wk, X', U, P
        "wy_prep_fused": (2 * dk + dv) * s + 4 + 4 * (C1 + 4.0) / C1 + 4 + dent
        + frags,
        # Wk, X', U, P, q -> o
        "wy_scan": frags + dk * s + dv * s,
        # q, k, b, v, w, log alpha -> Wk, X', U, P, Q^, exit decay
        "gdn2_prep": (3 * dk + 2 * dv) * s + 4 * dk + frags_g,
        # Wk, X', U, P, Q^, exit decay -> o
        "gdn2_scan": frags_g + dv * s,
        # q, k, k~, v, beta, log alpha -> Wk, X', U, P, Q^, exit decay
        "gated_prep": (3 * dk + dv) * s + 4 + 4 * dk + frags_g,
        "gated_scan": frags_g + dv * s,
        # q, k, v, beta, log alpha, log gate prefix, g, d entries -> Wk, X',
        # U, P, Q^, exit decay
        "gated_prep_fused": (2 * dk + dv) * s + 4 + 4 * dk
        + 4 * (C1 + 4.0) / C1 + 4 + dent + frags_g,
    }


def flops_per_token_head(w):
    """Chunk-form flops per token-head of phase 2: state chain 4 Dk Dv,
    inter-chunk output 2 Dk Dv, intra-chunk Gram, W and scores
    2 C (3 Dk + 2 Dv), triangular inverse about C^2 / 3."""
    C, dk, dv = w.chunk, w.Dk, w.Dv
    return 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3.0


LAUNCHES_PER_STEP = {}
COLD = None


def timed_steps(step, args):
    """Warm up, then time exactly args.steps steps (synchronised on both
    sides); returns the wall time per step (ms) and {kernel: ms per step}. The
    per-kernel durations come from a second pass of the same steps with the
    library's event timing on, so that the events do not weigh on the wall
    time."""
    import delta_rule_recurrent_scan_amd as osdn
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    osdn.kernel_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    osdn.kernel_timing(False)
    # per step: the summed duration of each kernel's launches (a kernel run
    # over time pieces launches several times per step)
    rec = osdn.kernel_times()
    kt = {n: ms * cnt / args.steps for n, (cnt, ms) in rec.items()}
    global LAUNCHES_PER_STEP, COLD
    LAUNCHES_PER_STEP = {n: cnt / args.steps for n, (cnt, ms) in rec.items()}
    COLD = cold_steps(step, args.steps)
    return wall * 1e3 / args.steps, kt


def cold_steps(step, n):
    """Each step timed alone (HIP events on the current stream) after 1 GiB
    of other data has been written, so that the memory-side cache and the L2
    no longer hold the step's inputs; returns median and min in ms."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    times = []
    for i in range(n):
        flush.fill_(float(i))
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    times.sort()
    return {"median_ms": times[len(times) // 2], "min_ms": times[0],
            "note": "each step timed alone after writing 1 GiB elsewhere "
                    "(inputs not in the memory-side cache or L2)"}


def roofline(w, kt, kb):
    """Roofline entry of the dominant (longest) kernel: its algorithmic bytes
    per step over its summed launch durations per step (= bytes per launch
    over the mean launch duration), against the HBM peak."""
    th = w.B * w.H * w.T
    dom = max(kt, key=lambda n: kt[n])
    n_l = LAUNCHES_PER_STEP.get(dom, 1.0)
    alg = kb[dom] * th / n_l
    achieved = alg / (kt[dom] / n_l * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": dom, "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(dom, w.name), "alg_bytes": alg,
            "ms": kt[dom] / n_l, "launches_per_step": n_l}


def cpu_baseline(w, inp, budget_s=12.0):
    """Time the fp64 oracle on whole (batch, head) streams until the budget is
    spent, then scale to the full workload (streams are independent)."""
    from oracle import recurrence as R
    f = W.to_f64
    q, k, v, beta = f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"])
    r = f(inp["r"]) if inp["r"] is not None else None
    done, t_used = 0, 0.0
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    while done < len(order) and t_used < budget_s:
        b, h = order[done]
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        R.osdn_ref(q[sl], k[sl], v[sl], beta[sl],
                   None if r is None else r[sl], inp["eta"])
        t_used += time.perf_counter() - t0
        done += 1
    per_stream = t_used / done
    total = per_stream * w.B * w.H
    return {"value": w.B * w.T / total, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of %d (batch, head) streams at full length T=%d, "
                      "fp64 NumPy token recurrence, one thread; scaled to all "
                      "streams" % (done, w.B * w.H, w.T)}


def bench_gated(args, w, inp, x, dt, dev):
    """One step = one osdn_gated_forward call (OSDN on a per-channel-decay
    backbone) over the workload."""
    import delta_rule_recurrent_scan_amd as osdn
    L = osdn.load_library()
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    S_T = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    d_T = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    ws_n = L.osdn_gated_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                                w.chunk, 1 if w.dtype == "bf16"
                                                else 0)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        osdn.osdn_gated_forward(x["q"], x["k"], x["v"], x["beta"],
                                x["log_alpha"], x["r"], x["eta"],
                                chunk=w.chunk, out=(o, S_T, d_T), workspace=ws)

    ms_step, kt = timed_steps(step, args)
    kb = kernel_bytes_per_token_head(w, inp["r"] is not None)
    rec = {
        "metric": "OSDN on a per-channel-decay backbone forward tokens/s + % "
                  "HBM roofline, H=16 d=128 T=4096, 1 GPU",
        "value": w.B * w.T / (ms_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T,
                   "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk},
        "roofline": roofline(w, kt, kb),
        "kernels_ms": kt,
        "cold_step": COLD,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_gated(w, inp)
    return rec


def cpu_baseline_gated(w, inp, budget_s=12.0):
    from oracle import recurrence as R
    f = W.to_f64
    arrs = {k: f(inp[k]) for k in ("q", "k", "v", "beta", "log_alpha", "r")}
    done, t_used = 0, 0.0
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    while done < len(order) and t_used < budget_s:
        b, h = order[done]
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        R.osdn_gated_ref(*(arrs[k][sl] for k in ("q", "k", "v", "beta",
                                                  "log_alpha", "r")), inp["eta"])
        t_used += time.perf_counter() - t0
        done += 1
    total = t_used / done * w.B * w.H
    return {"value": w.B * w.T / total, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of %d (batch, head) streams at full length T=%d, "
                      "fp64 NumPy token recurrence, one thread; scaled to all "
                      "streams" % (done, w.B * w.H, w.T)}


def bench_gdn2(args, w, inp, x, dt, dev):
    """One step = one gdn2_forward call over the workload."""
    import delta_rule_recurrent_scan_amd as osdn
    L = osdn.load_library()
    P = osdn._ptr
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    S_T = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    code = {torch.float32: 0, torch.bfloat16: 1}[dt]
    sp = torch.cuda.current_stream(dev).cuda_stream
    ws_n = L.gdn2_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk,
                                          code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        rc = L.gdn2_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code,
                            P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]),
                            P(x["b"]), P(x["w"]), None, 1.0, P(o), P(S_T),
                            P(ws), ws.numel(), sp)
        if rc:
            raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))

    ms_step, kt = timed_steps(step, args)
    kb = kernel_bytes_per_token_head(w)
    rec = {
        "metric": "GDN-2 forward tokens/s + % HBM roofline, H=16 d=128 "
                  "T=4096, 1 GPU",
        "value": w.B * w.T / (ms_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T,
                   "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk},
        "roofline": roofline(w, kt, kb),
        "kernels_ms": kt,
        "cold_step": COLD,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_gdn2(w, inp)
    return rec


def cpu_baseline_gdn2(w, inp, budget_s=12.0):
    from oracle import recurrence as R
    f = W.to_f64
    arrs = {k: f(inp[k]) for k in ("q", "k", "v", "log_alpha", "b", "w")}
    done, t_used = 0, 0.0
    order = [(b, h) for b in range(w.B) for h in range(w.H)]
    while done < len(order) and t_used < budget_s:
        b, h = order[done]
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        R.gdn2_ref(*(arrs[k][sl] for k in ("q", "k", "v", "log_alpha", "b", "w")))
        t_used += time.perf_counter() - t0
        done += 1
    total = t_used / done * w.B * w.H
    return {"value": w.B * w.T / total, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of %d (batch, head) streams at full length T=%d, "
                      "fp64 NumPy token recurrence, one thread; scaled to all "
                      "streams" % (done, w.B * w.H, w.T)}


def decode_bytes_per_head(w):
    """Algorithmic bytes per (batch, head) of one decode call: the fp32 state
    read and written once, plus the call's tokens (inputs and outputs) and,
    for OSDN, the preconditioner read and written."""
    s = 2 if w.dtype == "bf16" else 4
    state = 2 * w.Dk * w.Dv * 4
    if w.kind == "osdn":
        tok = (2 * w.Dk + w.Dv) * s + w.Dv * s + 4 + (4 if w.apf else 0)
        return state + 2 * w.Dk * 4 + w.T * tok
    tok = (3 * w.Dk + 2 * w.Dv) * s + 4 * w.Dk + w.Dv * s
    return state + w.T * tok


def bench_decode(args, w, inp, x, dt, dev):
    """One step = one recurrent decode call (w.T tokens for every (batch,
    head) stream) with the state updated in place."""
    import delta_rule_recurrent_scan_amd as osdn
    S = x["S0"].clone()
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    if w.kind == "osdn":
        d = x["d0"].clone()

        def step():
            osdn.osdn_decode(x["q"], x["k"], x["v"], x["beta"], S, d, r=x["r"],
                             eta=x["eta"], out=o)
    else:
        def step():
            osdn.gdn2_decode(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                             x["w"], S, out=o)
    ms_step, kt = timed_steps(step, args)
    name = "%s_decode" % w.kind
    alg = decode_bytes_per_head(w) * w.B * w.H
    achieved = alg / (kt[name] * 1e-3) / 1e9
    label = "OSDN" if w.kind == "osdn" else "GDN-2"
    rec = {
        "metric": "%s recurrent decode tokens/s + %% HBM roofline, B=%d H=%d "
                  "d=%d, 1 GPU" % (label, w.B, w.H, w.Dk),
        "value": w.B * w.T / (ms_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T,
                   "Dk": w.Dk, "Dv": w.Dv},
        "roofline": {"bound": "hbm", "kernel": name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name, w.name),
                     "alg_bytes": alg, "ms": kt[name]},
        "kernels_ms": kt,
        "cold_step": COLD,
        # back-to-back decode steps find much of the state in the memory-side
        # cache (the whole state of this workload fits in it); the cold step
        # (state and inputs evicted first, launch included) bounds the HBM rate
        "roofline_cold": {"achieved": alg / (COLD["median_ms"] * 1e-3) / 1e9,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": alg / (COLD["median_ms"] * 1e-3) / 1e9
                          / HBM_PEAK_GBS},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_decode(w, inp)
    return rec


def cpu_baseline_decode(w, inp, budget_s=12.0):
    """The fp64 oracle on the same decode call, repeated until the budget is
    spent (all streams at once, vectorised over (batch, head))."""
    from oracle import recurrence as R
    f = W.to_f64
    if w.kind == "osdn":
        args = [f(inp[k]) for k in ("q", "k", "v", "beta", "r")]
        run = lambda: R.osdn_ref(*args, inp["eta"], f(inp["d0"]), f(inp["S0"]))
    else:
        args = [f(inp[k]) for k in ("q", "k", "v", "log_alpha", "b", "w", "S0")]
        run = lambda: R.gdn2_ref(*args)
    n, t_used = 0, 0.0
    while t_used < budget_s and n < 50:
        t0 = time.perf_counter()
        run()
        t_used += time.perf_counter() - t0
        n += 1
    return {"value": w.B * w.T * n / t_used, "unit": "tokens/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d repetitions of the whole call (all %d streams, T=%d), "
                      "fp64 NumPy token recurrence vectorised over streams, "
                      "one thread" % (n, w.B * w.H, w.T)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="osdn-1.3b-apf",
                    choices=[w.name for w in W.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
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
        return

    import delta_rule_recurrent_scan_amd as osdn

    w = W.BY_NAME[args.workload]
    inp = W.make_inputs(w)
    dev = torch.device("cuda:0")
    x = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
         for k, v in inp.items()}
    dt = W.torch_dtype(w.dtype)
    if w.state:
        print(json.dumps(bench_decode(args, w, inp, x, dt, dev)), flush=True)
        return
    if w.kind == "gdn2":
        print(json.dumps(bench_gdn2(args, w, inp, x, dt, dev)), flush=True)
        return
    if w.decay:
        print(json.dumps(bench_gated(args, w, inp, x, dt, dev)), flush=True)
        return
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    S_T = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    d_T = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    L = osdn.load_library()
    code = {torch.float32: 0, torch.bfloat16: 1}[dt]
    sp = torch.cuda.current_stream(dev).cuda_stream
    P = osdn._ptr
    ws_n = L.osdn_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk,
                                          code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step():
        rc = L.osdn_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code, P(x["q"]),
                            P(x["k"]), P(x["v"]), P(x["beta"]), P(x["r"]),
                            float(x["eta"]), None, None, 1.0, P(o), P(S_T),
                            P(d_T), None, None, P(ws), ws.numel(), sp)
        if rc:
            raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))

    ms_step, kt = timed_steps(step, args)
    th = w.B * w.H * w.T
    apf = inp["r"] is not None
    kb = kernel_bytes_per_token_head(w, apf)
    path_b = path_bytes_per_token_head(w, apf)
    flops = flops_per_token_head(w) * th
    rec = {
        "metric": "OSDN forward tokens/s + % HBM/MFMA roofline, H=16 d=128 "
                  "T=4096, 1 GPU",
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
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T,
                   "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk,
                   "forgetting_gate": apf, "eta": w.eta},
        "roofline": roofline(w, kt, kb),
        "kernels_ms": kt,
        "cold_step": COLD,
        "path": {"alg_bytes": path_b * th,
                 "hbm_GBs": path_b * th / (ms_step * 1e-3) / 1e9,
                 "hbm_frac": path_b * th / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "chunk_form_TFLOPs": flops / (ms_step * 1e-3) / 1e12,
                 "mfma_frac": flops / (ms_step * 1e-3) / 1e12
                 / MFMA_BF16_PEAK_TFLOPS},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
