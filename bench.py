"""Benchmark of the OSDN forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward (phase 1 preconditioner scan + phase 2 chunked WY
delta rule) over the workload's synthetic batch, inputs resident in HBM,
outputs and workspace preallocated. The step issues exactly the two kernel
launches osdn_forward makes, through their own C-ABI entry points, with HIP
events recorded around each launch on the launch stream so that per-kernel
durations are measured live over the timed region.

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
    "osdn_precond_scan": ["precond_scan.hip"],
    "osdn_chunk": ["wy_chunk.hip"],
    "gdn2_chunk": ["wy_chunk.hip"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (scaled by the copy-kernel calibration), or None when
    they were taken on another workload or on kernel sources that have
    changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[kernel] + ["device_common.hpp", "launch.hpp"]:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    if rec.get("source_sha") != h.hexdigest()[:16] or rec.get("workload") != workload:
        return None
    return rec["bytes"]


def bytes_per_token_head(w, apf):
    """Algorithmic bytes per token-head of each kernel and of the whole path.

    Whole path: q, k (Dk each) and v (Dv) read, o (Dv) written, beta (and r)
    read. Phase 1 reads k, beta (r) and writes k~ (Dk); phase 2 reads q, k,
    k~, v, beta and writes o.
    """
    s = 2 if w.dtype == "bf16" else 4
    g = 4 + (4 if apf else 0)
    path = (2 * w.Dk + w.Dv) * s + w.Dv * s + g
    p1 = 2 * w.Dk * s + g
    p2 = (3 * w.Dk + w.Dv) * s + w.Dv * s + 4
    return path, p1, p2


def flops_per_token_head(w):
    """Chunk-form flops per token-head of phase 2: state chain 4 Dk Dv,
    inter-chunk output 2 Dk Dv, intra-chunk Gram, W and scores
    2 C (3 Dk + 2 Dv), triangular inverse about C^2 / 3."""
    C, dk, dv = w.chunk, w.Dk, w.Dv
    return 6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3.0


def gdn2_bytes_per_token_head(w):
    """q, k, b (Dk) and v, w (Dv) read in the storage dtype, log alpha (Dk)
    read in fp32, o (Dv) written."""
    s = 2 if w.dtype == "bf16" else 4
    return (3 * w.Dk + 2 * w.Dv) * s + 4 * w.Dk + w.Dv * s


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


def bench_gdn2(args, w, inp, x, dt, dev):
    """One step = one gdn2_forward launch over the workload."""
    import delta_rule_recurrent_scan_amd as osdn
    L = osdn.load_library()
    P = osdn._ptr
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    S_T = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    code = {torch.float32: 0, torch.bfloat16: 1}[dt]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    ws_n = L.gdn2_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk,
                                          code)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = L.gdn2_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code,
                            P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]),
                            P(x["b"]), P(x["w"]), None, 1.0, P(o), P(S_T),
                            P(ws), ws.numel(), sp)
        if ev is not None:
            ev[1].record(stream)
        if rc:
            raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    k_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    th = w.B * w.H * w.T
    alg = gdn2_bytes_per_token_head(w) * th
    achieved = alg / (k_ms * 1e-3) / 1e9
    rec = {
        "metric": "GDN-2 forward tokens/s + % HBM roofline, H=16 d=128 "
                  "T=4096, 1 GPU",
        "value": w.B * w.T / (ms_step * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T,
                   "Dk": w.Dk, "Dv": w.Dv, "chunk": w.chunk},
        "roofline": {"bound": "hbm", "kernel": "gdn2_chunk",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("gdn2_chunk", w.name)},
        "kernels_ms": {"gdn2_chunk": k_ms},
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
    if w.kind == "gdn2":
        print(json.dumps(bench_gdn2(args, w, inp, x, dt, dev)), flush=True)
        return
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=dt, device=dev)
    S_T = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=dev)
    d_T = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=dev)
    ktil = torch.empty((w.B, w.H, w.T, w.Dk), dtype=dt, device=dev)
    L = osdn.load_library()
    code = {torch.float32: 0, torch.bfloat16: 1}[dt]
    # one scratch buffer serves both entry points (phase-1 scratch is dead
    # when phase 2 starts)
    pws_n = max(L.osdn_precond_workspace_bytes(w.B, w.H, w.T, w.Dk, code),
                L.osdn_chunk_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                             w.chunk, code))
    pws = torch.empty(max(pws_n, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    P = osdn._ptr

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        rc = L.osdn_precond_scan(w.B, w.H, w.T, w.Dk, code, P(x["k"]),
                                 P(x["beta"]), P(x["r"]), float(x["eta"]), None,
                                 P(ktil), P(d_T), P(pws), pws.numel(), sp)
        if ev is not None:
            ev[1].record(stream)
        rc |= L.osdn_chunk_forward(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code,
                                   P(x["q"]), P(x["k"]), P(ktil), P(x["v"]),
                                   P(x["beta"]), None, 1.0, P(o), P(S_T),
                                   P(pws), pws.numel(), sp)
        if ev is not None:
            ev[2].record(stream)
        if rc:
            raise RuntimeError("launch failed: %s" % L.osdn_strerror(rc))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    k1 = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))  # ms
    k2 = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    th = w.B * w.H * w.T
    apf = inp["r"] is not None
    path_b, p1_b, p2_b = bytes_per_token_head(w, apf)
    kernels = {
        "osdn_precond_scan": {"ms": k1, "alg_bytes": p1_b * th},
        "osdn_chunk": {"ms": k2, "alg_bytes": p2_b * th},
    }
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    achieved = kernels[dom]["alg_bytes"] / (kernels[dom]["ms"] * 1e-3) / 1e9
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
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dom, w.name),
                     "alg_bytes": kernels[dom]["alg_bytes"]},
        "kernels_ms": {n: kernels[n]["ms"] for n in kernels},
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
