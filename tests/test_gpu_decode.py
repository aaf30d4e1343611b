"""GPU parity of the recurrent decode entry points (osdn_decode, gdn2_decode)
against the fp64 oracle's token recurrence, started from the same state.

The decode kernels run the token recurrence in fp32 with the state held in
registers, so the tolerances are the path's own (relative L2 over the
compared tensor): o and the final state <= 1e-4 with fp32 inputs and
<= 2e-2 with bf16 inputs (o is rounded to bf16), d <= 1e-5. The full decode
workloads are compared element by element: one token for 2048 streams is
cheap for the oracle.
"""
import numpy as np
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W
from oracle import recurrence as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
D_TOL = 1e-5
DEV = "cuda:0"
f64 = W.to_f64


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0)


def dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def osdn_gpu(inp):
    x = dev(inp)
    S, d = x["S0"].clone(), x["d0"].clone()
    o = osdn.osdn_decode(x["q"], x["k"], x["v"], x["beta"], S, d, r=x["r"],
                         eta=x["eta"])
    torch.cuda.synchronize()
    return f64(o), f64(S), f64(d)


def osdn_oracle(inp):
    g = lambda key: None if inp.get(key) is None else f64(inp[key])
    return R.osdn_ref(g("q"), g("k"), g("v"), g("beta"), g("r"), inp["eta"],
                      g("d0"), g("S0"))


def gdn2_gpu(inp):
    x = dev(inp)
    S = x["S0"].clone()
    o = osdn.gdn2_decode(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                         x["w"], S)
    torch.cuda.synchronize()
    return f64(o), f64(S)


def gdn2_oracle(inp):
    return R.gdn2_ref(*(f64(inp[k]) for k in ("q", "k", "v", "log_alpha", "b",
                                               "w", "S0")))


def check(got, ref, dtype, where):
    errs = [rel_l2(g, r) for g, r in zip(got, ref)]
    print("%s: rel_l2 %s" % (where, " ".join("%.3e" % e for e in errs)),
          flush=True)
    for g in got:
        assert np.all(np.isfinite(g))
    assert errs[0] <= TOL[dtype], "o rel L2 %.3e" % errs[0]
    assert errs[1] <= TOL[dtype], "state rel L2 %.3e" % errs[1]
    if len(errs) > 2:
        assert errs[2] <= D_TOL, "d rel L2 %.3e" % errs[2]


OSDN_CASES = [(dk, dv, T, dt, apf)
              for dk, dv in [(128, 128), (32, 64), (64, 32)]
              for T, dt, apf in [(1, "bf16", True), (5, "bf16", False),
                                 (3, "f32", True)]] + [(128, 64, 40, "f32", True)]


@pytest.mark.parametrize("dk,dv,T,dt,apf", OSDN_CASES,
                         ids=["dk%d-dv%d-T%d-%s-%s" % (c[0], c[1], c[2], c[3],
                                                       "apf" if c[4] else "nogate")
                              for c in OSDN_CASES])
def test_osdn_decode_small(dk, dv, T, dt, apf):
    w = W.BY_NAME["osdn-decode"].scaled(B=2, H=3, T=T, Dk=dk, Dv=dv, dtype=dt,
                                        apf=apf)
    inp = W.make_inputs(w)
    check(osdn_gpu(inp), osdn_oracle(inp), dt, "osdn decode %s" % (w,))


def test_osdn_decode_full_size():
    w = W.BY_NAME["osdn-decode"]
    inp = W.make_inputs(w)
    check(osdn_gpu(inp), osdn_oracle(inp), w.dtype, w.name)


def test_osdn_decode_continues_forward():
    """A prompt through osdn_forward, then tokens one at a time through
    osdn_decode, against the oracle over the whole sequence."""
    w = W.BY_NAME["osdn-1.3b-apf"].scaled(B=1, H=2, T=100)
    inp = W.make_inputs(w)
    x = dev(inp)
    cut = 93
    _, S, d = osdn.osdn_forward(x["q"][:, :, :cut].contiguous(),
                                x["k"][:, :, :cut].contiguous(),
                                x["v"][:, :, :cut].contiguous(),
                                x["beta"][:, :, :cut].contiguous(),
                                x["r"][:, :, :cut].contiguous(), x["eta"])
    outs = []
    for t in range(cut, w.T):
        sl = lambda a: a[:, :, t:t + 1].contiguous()
        outs.append(osdn.osdn_decode(sl(x["q"]), sl(x["k"]), sl(x["v"]),
                                     sl(x["beta"]), S, d, r=sl(x["r"]),
                                     eta=x["eta"]))
    torch.cuda.synchronize()
    ro, rS, rd = osdn_oracle(inp)
    check((f64(torch.cat(outs, dim=2)), f64(S), f64(d)),
          (ro[:, :, cut:], rS, rd), "bf16", "forward then decode")


def test_osdn_decode_zero_key_and_zero_tokens():
    w = W.BY_NAME["osdn-decode"].scaled(B=1, H=4, T=2)
    inp = W.make_inputs(w)
    k = inp["k"].clone()
    k[0, 1, 0] = 0
    k[0, 3, :] = 0
    inp["k"] = k
    check(osdn_gpu(inp), osdn_oracle(inp), "bf16", "zero keys")
    # T = 0: the state is left untouched, bit for bit
    w0 = w.scaled(T=0)
    inp0 = W.make_inputs(w0)
    o, S, d = osdn_gpu(inp0)
    assert o.shape == (1, 4, 0, w.Dv)
    assert np.array_equal(S, f64(inp0["S0"])) and np.array_equal(d, f64(inp0["d0"]))


def test_osdn_decode_rejects_state_aliasing_input():
    w = W.BY_NAME["osdn-decode"].scaled(B=1, H=1, T=1, Dk=32, Dv=32)
    x = dev(W.make_inputs(w))
    S = x["S0"].clone()
    with pytest.raises(osdn.OsdnError, match="overlaps"):
        osdn.osdn_decode(x["q"], x["k"], x["v"], x["beta"], S,
                         S.view(-1)[:32].view(1, 1, 32), r=x["r"])


GDN2_CASES = [(128, 128, 1, "bf16"), (128, 128, 4, "bf16"), (32, 64, 2, "f32"),
              (64, 32, 3, "bf16"), (64, 128, 1, "f32"), (128, 64, 40, "f32")]


@pytest.mark.parametrize("dk,dv,T,dt", GDN2_CASES,
                         ids=["dk%d-dv%d-T%d-%s" % c for c in GDN2_CASES])
def test_gdn2_decode_small(dk, dv, T, dt):
    w = W.BY_NAME["gdn2-decode"].scaled(B=2, H=3, T=T, Dk=dk, Dv=dv, dtype=dt)
    inp = W.make_inputs(w)
    check(gdn2_gpu(inp), gdn2_oracle(inp), dt, "gdn2 decode %s" % (w,))


def test_gdn2_decode_full_size():
    w = W.BY_NAME["gdn2-decode"]
    inp = W.make_inputs(w)
    check(gdn2_gpu(inp), gdn2_oracle(inp), w.dtype, w.name)


def test_gdn2_decode_continues_forward():
    w = W.BY_NAME["gdn2-1.3b"].scaled(B=1, H=2, T=80)
    inp = W.make_inputs(w)
    x = dev(inp)
    cut = 77
    pre = {k: x[k][:, :, :cut].contiguous()
           for k in ("q", "k", "v", "log_alpha", "b", "w")}
    _, S = osdn.gdn2_forward(pre["q"], pre["k"], pre["v"], pre["log_alpha"],
                             pre["b"], pre["w"])
    post = {k: x[k][:, :, cut:].contiguous()
            for k in ("q", "k", "v", "log_alpha", "b", "w")}
    o = osdn.gdn2_decode(post["q"], post["k"], post["v"], post["log_alpha"],
                         post["b"], post["w"], S)
    torch.cuda.synchronize()
    ro, rS = R.gdn2_ref(*(f64(inp[k]) for k in ("q", "k", "v", "log_alpha",
                                                 "b", "w")))
    check((f64(o), f64(S)), (ro[:, :, cut:], rS), "bf16", "gdn2 forward then decode")
