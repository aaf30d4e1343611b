"""GPU parity of OSDN on a per-key-channel-decay backbone (osdn_gated_forward,
and osdn_decode with a decay) against the fp64 oracle's token recurrence.

Tolerances as for OSDN (relative L2 over the compared tensor): o and S_T
<= 1e-4 on the fp32 path and <= 2e-2 on the bf16-input / fp32-state path,
d_T <= 1e-5.
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W
from oracle import recurrence as R
from parity import check_full

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
D_TOL = 1e-5
DEV = "cuda:0"
f64 = W.to_f64
BASE = W.BY_NAME["osdn-gated-1.3b"]


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0)


def dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def gpu(inp, chunk=None):
    x = dev(inp)
    o, S, d = osdn.osdn_gated_forward(x["q"], x["k"], x["v"], x["beta"],
                                      x["log_alpha"], x["r"], x["eta"],
                                      x.get("d0"), x.get("S0"),
                                      chunk=chunk or x["chunk"])
    torch.cuda.synchronize()
    return f64(o), f64(S), f64(d)


def oracle(inp, sl=(slice(None), slice(None))):
    g = lambda key: None if inp.get(key) is None else f64(inp[key])[sl]
    return R.osdn_gated_ref(g("q"), g("k"), g("v"), g("beta"), g("log_alpha"),
                            g("r"), inp["eta"], g("d0"), g("S0"))


def check(got, ref, dtype, where):
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    print("%s: rel_l2 o=%.3e S_T=%.3e d_T=%.3e" % ((where,) + tuple(errs)),
          flush=True)
    for a in got:
        assert np.all(np.isfinite(a))
    assert errs[0] <= TOL[dtype] and errs[1] <= TOL[dtype], errs
    assert errs[2] <= D_TOL, errs


SMALL = [
    BASE.scaled(B=1, H=2, T=64 * 3 + 21),
    BASE.scaled(B=2, H=1, T=100, chunk=32),
    BASE.scaled(B=1, H=2, T=77, Dk=64, Dv=128, chunk=16),
    BASE.scaled(B=1, H=2, T=90, Dk=128, Dv=64, apf=False),
    BASE.scaled(B=1, H=2, T=70, Dk=64, Dv=32, chunk=16, dtype="f32"),
    BASE.scaled(B=1, H=2, T=140, Dk=32, Dv=32, chunk=64, dtype="f32"),
    BASE.scaled(B=1, H=2, T=150, Dk=64, Dv=64, chunk=64, dtype="f32"),
    BASE.scaled(B=1, H=2, T=130, Dk=32, Dv=64, chunk=64),
    BASE.scaled(B=2, H=1, T=64, chunk=64),
    BASE.scaled(B=1, H=1, T=1, chunk=64),
]


@pytest.mark.parametrize("w", SMALL, ids=["T%d-C%d-dk%d-dv%d-%s" % (
    w.T, w.chunk, w.Dk, w.Dv, w.dtype) for w in SMALL])
def test_gated_small(w):
    if not osdn.load_library().osdn_gated_forward_supported(
            w.Dk, w.Dv, w.chunk, 1 if w.dtype == "bf16" else 0):
        pytest.skip("no kernel instance for this size")
    inp = W.make_inputs(w)
    check(gpu(inp), oracle(inp), w.dtype, "gated %s" % (w,))


def test_gated_scalar_decay_and_no_decay():
    """Equal channels (a Gated DeltaNet scalar decay), and no decay at all,
    which must agree with the plain OSDN forward."""
    w = BASE.scaled(B=1, H=2, T=150)
    inp = W.make_inputs(w)
    la = inp["log_alpha"]
    inp["log_alpha"] = la[..., :1].expand(la.shape).contiguous()
    check(gpu(inp), oracle(inp), "bf16", "scalar decay")
    inp["log_alpha"] = torch.zeros_like(la)
    got = gpu(inp)
    check(got, oracle(inp), "bf16", "no decay")
    ref = R.osdn_ref(*(f64(inp[k]) for k in ("q", "k", "v", "beta", "r")),
                     inp["eta"])
    check(got, ref, "bf16", "no decay vs plain OSDN oracle")


def test_gated_initial_state_in_place():
    w = BASE.scaled(B=1, H=2, T=130)
    inp = W.make_inputs(w)
    g = np.random.default_rng(31)
    S = torch.from_numpy((g.standard_normal((1, 2, w.Dv, w.Dk)) * 0.1)
                         .astype(np.float32))
    d = torch.from_numpy(g.uniform(0.5, 1.5, (1, 2, w.Dk)).astype(np.float32))
    inp["S0"], inp["d0"] = S, d
    ref = oracle(inp)
    x = dev(inp)
    Sd, dd = x["S0"].clone(), x["d0"].clone()
    o = torch.empty((1, 2, w.T, w.Dv), dtype=torch.bfloat16, device=DEV)
    osdn.osdn_gated_forward(x["q"], x["k"], x["v"], x["beta"], x["log_alpha"],
                            x["r"], x["eta"], dd, Sd, out=(o, Sd, dd))
    torch.cuda.synchronize()
    check((f64(o), f64(Sd), f64(dd)), ref, "bf16", "in place")


def test_gated_full_size_all_streams():
    w = BASE
    inp = W.make_inputs(w)
    o, S, d = gpu(inp)
    ro, rS, rd = oracle(inp)
    check_full("gated full size", w.dtype, o, ro, S, rS, d, rd)


def test_gated_decode_continues_forward():
    w = BASE.scaled(B=1, H=2, T=90)
    inp = W.make_inputs(w)
    x = dev(inp)
    cut = 85
    pre = {k: x[k][:, :, :cut].contiguous()
           for k in ("q", "k", "v", "beta", "r", "log_alpha")}
    _, S, d = osdn.osdn_gated_forward(pre["q"], pre["k"], pre["v"], pre["beta"],
                                      pre["log_alpha"], pre["r"], x["eta"])
    post = {k: x[k][:, :, cut:].contiguous()
            for k in ("q", "k", "v", "beta", "r", "log_alpha")}
    o = osdn.osdn_decode(post["q"], post["k"], post["v"], post["beta"], S, d,
                         r=post["r"], eta=x["eta"], log_alpha=post["log_alpha"])
    torch.cuda.synchronize()
    ro, rS, rd = oracle(inp)
    check((f64(o), f64(S), f64(d)), (ro[:, :, cut:], rS, rd), "bf16",
          "gated forward then decode")


@pytest.mark.parametrize("chunk,dtype", [(64, "bf16"), (16, "bf16"), (64, "f32")])
def test_gated_strong_decay(chunk, dtype):
    """OSDN on a decaying backbone with strong decays (log alpha = -2
    everywhere; random in (-6, 0); blocks at -8 that take the exact
    diagonal sums), at the fused chunk 64 and the materialised-K~ chunk 16."""
    dk, dv = (128, 128) if dtype == "bf16" else (32, 32)
    w = BASE.scaled(B=1, H=2, T=64 * 3 + 9, chunk=chunk, dtype=dtype, Dk=dk,
                    Dv=dv)
    inp = W.make_inputs(w)
    la0 = inp["log_alpha"]
    g = np.random.default_rng(12)
    mixed = la0.clone()
    for t0 in (16, 80, 144):
        mixed[:, :, t0:t0 + 16] = -8.0
    cases = [("log alpha = -2", torch.full_like(la0, -2.0)),
             ("log alpha in (-6, 0)",
              torch.from_numpy((-6.0 * g.random(la0.shape)).astype(np.float32))),
             ("blocks at -8", mixed)]
    for name, la in cases:
        inp["log_alpha"] = la
        check(gpu(inp), oracle(inp), dtype, "%s C=%d %s" % (name, chunk, dtype))
