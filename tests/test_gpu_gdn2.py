"""GPU parity of the HIP Gated DeltaNet-2 forward against the fp64 oracle.

Relative L2 tolerances as for OSDN: <= 1e-4 on the fp32 path and <= 2e-2 on
the bf16-input / fp32-state path, for o and S_T.
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
DEV = "cuda:0"


def rel_l2(x, ref):
    den = np.linalg.norm(ref)
    return np.linalg.norm(np.asarray(x, np.float64) - ref) / (den if den > 0 else 1.0)


def run(inp, chunk=None, scale=1.0, S0=None):
    x = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    S0d = None if S0 is None else S0.to(DEV)
    o, S = osdn.gdn2_forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                             x["w"], S0d, chunk=chunk or x["chunk"], scale=scale)
    torch.cuda.synchronize()
    return W.to_f64(o), W.to_f64(S)


def oracle(inp, sl=(slice(None), slice(None)), scale=1.0, S0=None):
    f = lambda key: W.to_f64(inp[key])[sl]
    s0 = None if S0 is None else W.to_f64(S0)[sl]
    return R.gdn2_ref(f("q"), f("k"), f("v"), f("log_alpha"), f("b"), f("w"),
                      s0, scale)


def check(got, ref, dtype, where):
    eo, eS = rel_l2(got[0], ref[0]), rel_l2(got[1], ref[1])
    print("%s: rel_l2 o=%.3e S_T=%.3e" % (where, eo, eS), flush=True)
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[1]))
    assert eo <= TOL[dtype], "o rel L2 %.3e" % eo
    assert eS <= TOL[dtype], "S_T rel L2 %.3e" % eS


BASE = W.BY_NAME["gdn2-1.3b"]
SMALL = [
    BASE.scaled(B=1, H=2, T=64 * 4 + 19),
    BASE.scaled(B=2, H=1, T=100, chunk=32),
    BASE.scaled(B=1, H=2, T=77, chunk=16, Dk=32, Dv=64),
    BASE.scaled(B=1, H=2, T=90, Dk=64, Dv=32, chunk=32),
    BASE.scaled(B=1, H=2, T=120, dtype="f32", Dk=32, Dv=32, chunk=16),
    BASE.scaled(B=1, H=2, T=70, dtype="f32", Dk=64, Dv=32, chunk=32),
    # around one chunk: a single token, exactly one chunk, one token past it
    BASE.scaled(B=1, H=2, T=1),
    BASE.scaled(B=1, H=2, T=64),
    BASE.scaled(B=1, H=2, T=65),
]


@pytest.mark.parametrize("w", SMALL, ids=["%s-T%d-dk%d-dv%d-c%d-%s" % (
    w.name, w.T, w.Dk, w.Dv, w.chunk, w.dtype) for w in SMALL])
def test_gdn2_parity_small(w):
    if not osdn.load_library().gdn2_forward_supported(
            w.Dk, w.Dv, w.chunk, 1 if w.dtype == "bf16" else 0):
        pytest.skip("no kernel instance for this size")
    inp = W.make_inputs(w)
    check(run(inp), oracle(inp), w.dtype, w.name)


def test_gdn2_initial_state_scale_and_chunks():
    w = BASE.scaled(B=1, H=2, T=150)
    inp = W.make_inputs(w)
    g = np.random.default_rng(3)
    S0 = torch.from_numpy(g.standard_normal((1, 2, w.Dk, w.Dv)).astype(np.float32) * 0.2)
    ref = oracle(inp, scale=0.5, S0=S0)
    for c in (16, 32, 64):
        check(run(inp, chunk=c, scale=0.5, S0=S0), ref, "bf16", "C=%d" % c)


def test_gdn2_reduces_to_deltanet():
    """b = w = beta and alpha = 1: GDN-2 equals DeltaNet with the state
    transposed; compared with the oracle's DeltaNet and with the GPU OSDN
    path at d = 1, eta = 0."""
    w = W.BY_NAME["osdn-340m"].scaled(B=1, H=2, T=140)
    x = W.make_inputs(w)
    beta = x["beta"]
    inp = dict(q=x["q"], k=x["k"], v=x["v"], chunk=64,
               log_alpha=torch.zeros(x["k"].shape, dtype=torch.float32),
               b=beta[..., None].expand(x["k"].shape).to(torch.bfloat16).contiguous(),
               w=beta[..., None].expand(x["v"].shape).to(torch.bfloat16).contiguous())
    o, S = run(inp)
    # the gates were rounded to bf16: the oracle gets the same rounded values
    f = W.to_f64
    ro, rS = R.gdn2_ref(f(inp["q"]), f(inp["k"]), f(inp["v"]),
                        np.zeros(x["k"].shape), f(inp["b"]), f(inp["w"]))
    assert rel_l2(o, ro) < 2e-2 and rel_l2(S, rS) < 2e-2
    dn_o, dn_S = R.deltanet_ref(f(x["q"]), f(x["k"]), f(x["v"]), f(beta))
    assert rel_l2(o, dn_o) < 2e-2
    assert rel_l2(S, np.swapaxes(dn_S, -1, -2)) < 2e-2


def test_gdn2_empty_sequence():
    w = BASE.scaled(B=1, H=2, T=0)
    inp = W.make_inputs(w)
    S0 = torch.randn((1, 2, w.Dk, w.Dv))
    o, S = run(inp, S0=S0)
    assert o.shape == (1, 2, 0, w.Dv)
    assert np.array_equal(S, W.to_f64(S0))


def test_gdn2_full_size_all_streams():
    w = BASE
    inp = W.make_inputs(w)
    o, S = run(inp)
    ro, rS = oracle(inp)
    check_full("gdn2 full size", "bf16", o, ro, S, rS)


def _decay_cases(w, seed):
    """Strong decays: log alpha = -2 on every token and channel (a chunk of
    64 sums to -128); log alpha in (-6, 0) at random; and -8 on the tokens
    of a few 16-token blocks (a block decays by e^-120 there, so its
    diagonal tile is summed element by element) with the workload's decay
    elsewhere."""
    la0 = W.make_inputs(w)["log_alpha"]
    g = np.random.default_rng(seed)
    strong = torch.full_like(la0, -2.0)
    rand = torch.from_numpy((-6.0 * g.random(la0.shape)).astype(np.float32))
    mixed = la0.clone()
    for t0 in (16, 80, 144):
        if t0 < w.T:
            mixed[:, :, t0:t0 + 16] = -8.0
    mixed[:, 1:, :, : w.Dk // 2] = -8.0     # half the channels of head 1
    return [("log alpha = -2", strong), ("log alpha in (-6, 0)", rand),
            ("blocks at -8", mixed)]


@pytest.mark.parametrize("chunk,dtype", [(64, "bf16"), (32, "bf16"), (16, "bf16"),
                                         (16, "f32"), (64, "f32")])
def test_gdn2_strong_decay(chunk, dtype):
    """Any log alpha <= 0: the in-chunk decay is split at 16-token blocks so
    every factor stays finite; the GPU matches the oracle to the usual
    bound (decays too strong for the factored diagonal are summed exactly)."""
    dk, dv = (128, 128) if dtype == "bf16" else (32, 32)
    w = BASE.scaled(B=1, H=2, T=64 * 3 + 9, chunk=chunk, dtype=dtype, Dk=dk,
                    Dv=dv)
    if not osdn.load_library().gdn2_forward_supported(
            dk, dv, chunk, 1 if dtype == "bf16" else 0):
        pytest.skip("no kernel instance for this size")
    inp = W.make_inputs(w)
    for name, la in _decay_cases(w, 11):
        inp["log_alpha"] = la
        check(run(inp), oracle(inp), dtype, "%s C=%d %s" % (name, chunk, dtype))
