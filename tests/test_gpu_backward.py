"""GPU parity of the OSDN backward (osdn_backward) against the fp64 oracle
adjoint (oracle.backward.osdn_backward_ref), which the CPU tests pin to
central differences of the forward oracle.

The backward runs the recurrence and its adjoint in fp32 on inputs that the
oracle sees bit for bit (bf16 inputs widened exactly), and writes fp32
gradients, so the differences are fp32 rounding only, also for bf16 inputs:
the bar is the fp32 path's, a relative L2 error of 1e-4 over every gradient
tensor and over every (batch, head) stream of it on its own. Oracle-sized
cases compare every element (several 64-token checkpoint intervals and a
ragged tail); the full 1.3B-layer workload compares sampled streams, which
the oracle computes one at a time at full length.
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W
from oracle.backward import osdn_backward_ref
from parity import per_stream_rel_l2, rel_l2

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 1e-4
NAMES = ("q", "k", "v", "beta", "r", "eta", "d0", "S0")
f64 = W.to_f64


def to_dev(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in x.items()}


def gpu_backward(inp, cot, scale=1.0):
    x, c = to_dev(inp), to_dev(cot)
    g = osdn.osdn_backward(x["q"], x["k"], x["v"], x["beta"], c["do"],
                           r=x["r"], eta=x["eta"], d0=x.get("d0"),
                           S0=x.get("S0"), dS_T=c["dS_T"], dd_T=c["dd_T"],
                           scale=scale)
    torch.cuda.synchronize()
    return {n: f64(g[n]) for n in NAMES}


def oracle_backward(inp, cot, scale=1.0):
    g = lambda d, key: None if d.get(key) is None else f64(d[key])
    return osdn_backward_ref(g(inp, "q"), g(inp, "k"), g(inp, "v"),
                             g(inp, "beta"), g(inp, "r"), inp["eta"],
                             g(inp, "d0"), g(inp, "S0"), g(cot, "do"),
                             g(cot, "dS_T"), g(cot, "dd_T"), scale=scale)


def check(where, got, ref, tol=TOL):
    msg = []
    ok = True
    for n in NAMES:
        assert got[n].shape == ref[n].shape, n
        assert np.all(np.isfinite(got[n])), "%s: non-finite d%s" % (where, n)
        e = rel_l2(got[n], ref[n])
        s = per_stream_rel_l2(got[n], ref[n]).max() if got[n].size else 0.0
        msg.append("d%s %.2e/%.2e" % (n, e, s))
        ok = ok and e <= tol and s <= tol
    line = "%s: rel_l2 (tensor/worst stream) %s" % (where, " ".join(msg))
    print(line, flush=True)
    assert ok, line


def wl(name, **kw):
    return W.BY_NAME[name].scaled(**kw)


CASES = [
    # (id, workload, scale, cotangents of S_T and d_T)
    ("tiny-fp32", W.BY_NAME["tiny-fp32"], 1.0, True),
    ("tiny-fp32-o-only", W.BY_NAME["tiny-fp32"], 1.0, False),
    ("1.3b-apf-T300", wl("osdn-1.3b-apf", B=1, H=2, T=300), 1.0, True),
    ("1.3b-apf-T300-scaled", wl("osdn-1.3b-apf", B=1, H=2, T=300),
     128 ** -0.5, False),
    ("340m-T129", wl("osdn-340m", B=2, H=1, T=129), 1.0, True),
    ("recall-T200", wl("osdn-recall-8k", B=1, H=2, T=200), 1.0, True),
    ("state-T150", wl("osdn-decode", B=2, H=2, T=150), 1.0, True),
    ("T1", wl("osdn-1.3b-apf", B=2, H=1, T=1), 1.0, True),
    ("T64", wl("osdn-1.3b-apf", B=1, H=1, T=64), 1.0, True),
    ("T65", wl("osdn-1.3b-apf", B=1, H=1, T=65), 1.0, True),
] + [
    ("dk%d-dv%d-%s" % (dk, dv, dt),
     wl("tiny-fp32", B=2, H=1, T=70, Dk=dk, Dv=dv, dtype=dt, apf=True,
        state=True), 1.0, True)
    for dk, dv in ((32, 64), (64, 32), (128, 32), (64, 128), (32, 128))
    for dt in ("f32", "bf16")
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(case):
    name, w, scale, state = case
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w, state=state)
    check(name, gpu_backward(inp, cot, scale), oracle_backward(inp, cot, scale))


def test_backward_zero_keys():
    """Tokens with an all-zero key: the learner takes no step there and no
    gradient flows through its step size (the forward's convention)."""
    w = wl("osdn-1.3b-apf", B=1, H=2, T=150, state=True)
    inp = W.make_inputs(w)
    k = inp["k"].clone()
    k[:, :, [0, 63, 64, 100, 149]] = 0
    inp["k"] = k
    cot = W.make_cotangents(w)
    got, ref = gpu_backward(inp, cot), oracle_backward(inp, cot)
    check("zero keys", got, ref)
    # no key, no write: the value and beta gradients vanish exactly there
    for t in (0, 63, 64, 100, 149):
        assert np.all(got["v"][:, :, t] == 0.0)
        assert np.all(got["beta"][:, :, t] == 0.0)


@pytest.mark.parametrize("state", [True, False])
def test_backward_no_tokens(state):
    """T = 0: the gradients of S0 and d0 are the output adjoints themselves
    (zero when absent), eta's is zero."""
    w = wl("osdn-1.3b-apf", B=2, H=3, T=0, state=True)
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w, state=state)
    got = gpu_backward(inp, cot)
    zS = np.zeros((2, 3, 128, 128))
    zd = np.zeros((2, 3, 128))
    assert np.array_equal(got["S0"], f64(cot["dS_T"]) if state else zS)
    assert np.array_equal(got["d0"], f64(cot["dd_T"]) if state else zd)
    assert np.array_equal(got["eta"], np.zeros((2, 3)))
    for n in ("q", "k", "v", "beta", "r"):
        assert got[n].size == 0


def test_backward_full_size_sampled_streams():
    """The 1.3B-layer workload (4 x 16 streams x 4096 tokens, bf16, gate on)
    in one launch; two sampled streams against the oracle at full length,
    every stream finite."""
    w = W.BY_NAME["osdn-1.3b-apf"]
    inp = W.make_inputs(w)
    cot = W.make_cotangents(w)
    x, c = to_dev(inp), to_dev(cot)
    g = osdn.osdn_backward(x["q"], x["k"], x["v"], x["beta"], c["do"],
                           r=x["r"], eta=x["eta"], dS_T=c["dS_T"],
                           dd_T=c["dd_T"])
    torch.cuda.synchronize()
    for n in NAMES:
        assert bool(torch.isfinite(g[n]).all()), n
    for b, h in ((0, 0), (3, 13)):
        sl = lambda t: None if t is None else t[b:b + 1, h:h + 1].contiguous()
        si = {k: (sl(v) if isinstance(v, torch.Tensor) or v is None else v)
              for k, v in inp.items()}
        sc = {k: sl(v) for k, v in cot.items()}
        ref = oracle_backward(si, sc)
        got = {n: f64(g[n][b:b + 1, h:h + 1]) for n in NAMES}
        check("1.3b full, stream (%d, %d)" % (b, h), got, ref)
        del ref
