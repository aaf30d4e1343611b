"""GPU parity of the gate-aware backward passes (gdn2_backward and
osdn_gated_backward) against the fp64 oracle adjoints
(oracle.backward.gdn2_backward_ref, osdn_gated_backward_ref), which the CPU
tests pin to central differences of gdn2_ref and osdn_gated_ref.

As for the plain backward, the GPU runs the recurrence and its adjoint in
fp32 on inputs the oracle sees bit for bit and writes fp32 gradients: the
bar is the fp32 path's relative L2 error of 1e-4, over every gradient tensor
and every (batch, head) stream of it. The cases span several 64-token
recompute intervals and a ragged tail, strong decays (log alpha = -2 on
every token, random in (-6, 0), blocks at -8), drawn initial states, mixed
head dims, T = 0, 1, 64, 65, and sampled streams of the full 1.3B-layer
workloads.
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W
from oracle.backward import gdn2_backward_ref, osdn_gated_backward_ref
from parity import per_stream_rel_l2, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4
G2_NAMES = ("q", "k", "v", "log_alpha", "b", "w", "S0")
OG_NAMES = ("q", "k", "v", "beta", "r", "eta", "log_alpha", "d0", "S0")
f64 = W.to_f64


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


def opt(d, key):
    return None if d.get(key) is None else f64(d[key])


def gdn2_gpu(inp, cot, scale=1.0):
    x, c = to_dev(inp), to_dev(cot)
    g = osdn.gdn2_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                           x["w"], c["do"], S0=x.get("S0"), dS_T=c["dS_T"],
                           scale=scale)
    torch.cuda.synchronize()
    return {n: f64(g[n]) for n in G2_NAMES}


def gdn2_oracle(inp, cot, scale=1.0):
    return gdn2_backward_ref(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                             f64(inp["log_alpha"]), f64(inp["b"]),
                             f64(inp["w"]), opt(inp, "S0"), f64(cot["do"]),
                             opt(cot, "dS_T"), scale=scale)


def gated_gpu(inp, cot, scale=1.0):
    x, c = to_dev(inp), to_dev(cot)
    g = osdn.osdn_gated_backward(x["q"], x["k"], x["v"], x["beta"],
                                 x["log_alpha"], c["do"], r=x["r"],
                                 eta=x["eta"], d0=x.get("d0"), S0=x.get("S0"),
                                 dS_T=c["dS_T"], dd_T=c["dd_T"], scale=scale)
    torch.cuda.synchronize()
    return {n: f64(g[n]) for n in OG_NAMES}


def gated_oracle(inp, cot, scale=1.0):
    return osdn_gated_backward_ref(
        f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["beta"]),
        f64(inp["log_alpha"]), opt(inp, "r"), inp["eta"], opt(inp, "d0"),
        opt(inp, "S0"), f64(cot["do"]), opt(cot, "dS_T"), opt(cot, "dd_T"),
        scale=scale)


def check(where, got, ref, names, tol=TOL):
    msg, ok = [], True
    for n in names:
        assert got[n].shape == ref[n].shape, n
        assert np.all(np.isfinite(got[n])), "%s: non-finite d%s" % (where, n)
        e = rel_l2(got[n], ref[n])
        s = per_stream_rel_l2(got[n], ref[n]).max() if got[n].size else 0.0
        msg.append("d%s %.2e/%.2e" % (n, e, s))
        ok = ok and e <= tol and s <= tol
    line = "%s: rel_l2 (tensor/worst stream) %s" % (where, " ".join(msg))
    print(line, flush=True)
    assert ok, line


def decay_cases(w, seed):
    """log alpha = -2 everywhere; random in (-6, 0); blocks of 16 tokens and
    half the channels of one head at -8, the workload's decay elsewhere."""
    la0 = W.make_inputs(w)["log_alpha"]
    g = np.random.default_rng(seed)
    strong = torch.full_like(la0, -2.0)
    rand = torch.from_numpy((-6.0 * g.random(la0.shape)).astype(np.float32))
    mixed = la0.clone()
    for t0 in (16, 80, 144):
        if t0 < w.T:
            mixed[:, :, t0:t0 + 16] = -8.0
    mixed[:, 1:, :, : w.Dk // 2] = -8.0
    return [("log alpha = -2", strong), ("log alpha in (-6, 0)", rand),
            ("blocks at -8", mixed)]


G2 = W.BY_NAME["gdn2-1.3b"]
OG = W.BY_NAME["osdn-gated-1.3b"]


def g2_cases():
    return [
        ("1.3b-T300", G2.scaled(B=1, H=2, T=300), 1.0, True),
        ("1.3b-T300-o-only-scaled", G2.scaled(B=1, H=2, T=300), 128 ** -0.5,
         False),
        ("state-T150", W.BY_NAME["gdn2-decode"].scaled(B=2, H=2, T=150), 1.0,
         True),
        ("T1", G2.scaled(B=2, H=1, T=1), 1.0, True),
        ("T64", G2.scaled(B=1, H=1, T=64), 1.0, True),
        ("T65", G2.scaled(B=1, H=1, T=65), 1.0, True),
    ] + [("dk%d-dv%d-%s" % (dk, dv, dt),
          G2.scaled(B=2, H=1, T=70, Dk=dk, Dv=dv, dtype=dt, state=True), 1.0,
          True)
         for dk, dv in ((32, 64), (64, 32), (128, 32), (32, 128))
         for dt in ("f32", "bf16")]


def og_cases():
    return [
        ("1.3b-T300", OG.scaled(B=1, H=2, T=300), 1.0, True),
        ("1.3b-T300-o-only-scaled", OG.scaled(B=1, H=2, T=300), 128 ** -0.5,
         False),
        ("state-T150", OG.scaled(B=2, H=2, T=150, state=True), 1.0, True),
        ("no-gate-T129", OG.scaled(B=2, H=1, T=129, apf=False), 1.0, True),
        ("T1", OG.scaled(B=2, H=1, T=1), 1.0, True),
        ("T64", OG.scaled(B=1, H=1, T=64), 1.0, True),
        ("T65", OG.scaled(B=1, H=1, T=65), 1.0, True),
    ] + [("dk%d-dv%d-%s" % (dk, dv, dt),
          OG.scaled(B=2, H=1, T=70, Dk=dk, Dv=dv, dtype=dt, state=True), 1.0,
          True)
         for dk, dv in ((32, 64), (64, 32), (128, 32), (32, 128))
         for dt in ("f32", "bf16")]


@pytest.mark.parametrize("case", g2_cases(), ids=[c[0] for c in g2_cases()])
def test_gdn2_backward_parity(case):
    name, w, scale, state = case
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w, state=state)
    check("gdn2 " + name, gdn2_gpu(inp, cot, scale), gdn2_oracle(inp, cot, scale),
          G2_NAMES)


@pytest.mark.parametrize("case", og_cases(), ids=[c[0] for c in og_cases()])
def test_gated_backward_parity(case):
    name, w, scale, state = case
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w, state=state)
    check("gated " + name, gated_gpu(inp, cot, scale),
          gated_oracle(inp, cot, scale), OG_NAMES)


@pytest.mark.parametrize("kind", ["gdn2", "gated"])
def test_backward_strong_decay(kind):
    base = G2 if kind == "gdn2" else OG
    w = base.scaled(B=1, H=2, T=64 * 3 + 9, state=True)
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w)
    for name, la in decay_cases(w, 12):
        inp["log_alpha"] = la
        if kind == "gdn2":
            check("gdn2 " + name, gdn2_gpu(inp, cot), gdn2_oracle(inp, cot),
                  G2_NAMES)
        else:
            check("gated " + name, gated_gpu(inp, cot), gated_oracle(inp, cot),
                  OG_NAMES)


def test_gated_backward_zero_keys():
    w = OG.scaled(B=1, H=2, T=150, state=True)
    inp = W.make_inputs(w)
    k = inp["k"].clone()
    k[:, :, [0, 63, 64, 100, 149]] = 0
    inp["k"] = k
    cot = W.make_cotangents(w)
    got = gated_gpu(inp, cot)
    check("gated zero keys", got, gated_oracle(inp, cot), OG_NAMES)
    for t in (0, 63, 64, 100, 149):
        assert np.all(got["v"][:, :, t] == 0.0)


@pytest.mark.parametrize("kind", ["gdn2", "gated"])
def test_backward_no_tokens(kind):
    """T = 0: S0's gradient is dS_T itself (d0's is dd_T), eta's zero."""
    base = G2 if kind == "gdn2" else OG
    w = base.scaled(B=2, H=3, T=0, Dk=64, Dv=32, state=True)
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w)
    if kind == "gdn2":
        got = gdn2_gpu(inp, cot)
        assert np.array_equal(got["S0"], f64(cot["dS_T"]))
        names = ("q", "k", "v", "log_alpha", "b", "w")
    else:
        got = gated_gpu(inp, cot)
        assert np.array_equal(got["S0"], f64(cot["dS_T"]))
        assert np.array_equal(got["d0"], f64(cot["dd_T"]))
        assert np.array_equal(got["eta"], np.zeros((2, 3)))
        names = ("q", "k", "v", "beta", "r", "log_alpha")
    for n in names:
        assert got[n].size == 0


@pytest.mark.parametrize("kind", ["gdn2", "gated"])
def test_backward_full_size_sampled_streams(kind):
    """The 1.3B-layer workload (4 x 16 streams x 4096 tokens, bf16) in one
    launch; two sampled streams against the oracle at full length, every
    stream finite."""
    w = G2 if kind == "gdn2" else OG
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w)
    run = gdn2_gpu if kind == "gdn2" else gated_gpu
    ref_fn = gdn2_oracle if kind == "gdn2" else gated_oracle
    names = G2_NAMES if kind == "gdn2" else OG_NAMES
    got_all = run(inp, cot)
    for n in names:
        assert np.all(np.isfinite(got_all[n])), n
    for b, h in ((0, 0), (3, 13)):
        sl = lambda t: None if t is None else t[b:b + 1, h:h + 1].contiguous()
        si = {k: (sl(v) if isinstance(v, torch.Tensor) or v is None else v)
              for k, v in inp.items()}
        sc = {k: sl(v) for k, v in cot.items()}
        got = {n: got_all[n][b:b + 1, h:h + 1] for n in names}
        check("%s 1.3b full, stream (%d, %d)" % (kind, b, h), got,
              ref_fn(si, sc), names)
