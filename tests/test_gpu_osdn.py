"""GPU parity of the HIP OSDN forward against the fp64 CPU oracle.

Tolerances (relative L2 over the compared tensor, ||x - ref|| / ||ref||):
o and S_T <= 1e-4 on the fp32 path and <= 2e-2 on the bf16-input / fp32-state
path; d_T <= 1e-5 on both. Oracle-sized cases compare every element; the full
workload sizes compare sampled (batch, head) streams, which the oracle
computes independently at full length.
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


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(x - ref) / (den if den > 0 else 1.0)


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def gpu_forward(inp, chunk=None, **kw):
    x = to_dev(inp)
    args = dict(r=x["r"], eta=x["eta"], d0=x.get("d0"), S0=x.get("S0"),
                chunk=chunk or x["chunk"])
    args.update(kw)
    o, S, d = osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"], **args)
    torch.cuda.synchronize()
    return W.to_f64(o), W.to_f64(S), W.to_f64(d)


def oracle(inp, sl=(slice(None), slice(None)), scale=1.0):
    f = lambda key: None if inp.get(key) is None else W.to_f64(inp[key])[sl]
    return R.osdn_ref(f("q"), f("k"), f("v"), f("beta"), f("r"), inp["eta"],
                      f("d0"), f("S0"), scale)


def check(got, ref, dtype, where):
    o, S, d = got
    ro, rS, rd = ref
    eo, eS, ed = rel_l2(o, ro), rel_l2(S, rS), rel_l2(d, rd)
    print("%s: rel_l2 o=%.3e S_T=%.3e d_T=%.3e" % (where, eo, eS, ed), flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[dtype], "o rel L2 %.3e" % eo
    assert eS <= TOL[dtype], "S_T rel L2 %.3e" % eS
    assert ed <= D_TOL, "d_T rel L2 %.3e" % ed


def small(name, **kw):
    w = W.BY_NAME[name]
    return w.scaled(**kw)


# Oracle-sized versions of every OSDN workload: several chunks plus a ragged
# tail (T not a multiple of the chunk).
SMALL = [
    W.BY_NAME["tiny-fp32"],
    small("tiny-fp32", T=16 * 5 + 9),
    small("osdn-340m", B=1, H=2, T=64 * 4 + 35),
    small("osdn-1.3b-apf", B=2, H=1, T=64 * 3 + 17),
    small("osdn-recall-8k", B=1, H=2, T=64 * 5 + 1),
]


@pytest.mark.parametrize("w", SMALL, ids=["%s-T%d" % (w.name, w.T) for w in SMALL])
def test_parity_small(w):
    inp = W.make_inputs(w)
    check(gpu_forward(inp), oracle(inp), w.dtype, w.name)


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_invariance(chunk):
    w = small("osdn-1.3b-apf", B=1, H=2, T=200)
    inp = W.make_inputs(w)
    check(gpu_forward(inp, chunk=chunk), oracle(inp), w.dtype, "C=%d" % chunk)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 64), (32, 128),
                                   (128, 32)])
def test_head_dims_bf16(dk, dv):
    w = small("osdn-1.3b-apf", B=1, H=3, T=150, Dk=dk, Dv=dv)
    inp = W.make_inputs(w)
    check(gpu_forward(inp), oracle(inp), "bf16", "dk=%d dv=%d" % (dk, dv))


@pytest.mark.parametrize("dk,dv,chunk", [(32, 32, 16), (64, 32, 32),
                                         (32, 64, 32), (64, 64, 16)])
def test_head_dims_fp32(dk, dv, chunk):
    if not osdn.supported(dk, dv, chunk, torch.float32):
        pytest.skip("no fp32 kernel instance for this size")
    w = small("tiny-fp32", B=1, H=2, T=100, Dk=dk, Dv=dv, chunk=chunk)
    inp = W.make_inputs(w)
    check(gpu_forward(inp), oracle(inp), "f32", "fp32 dk=%d dv=%d" % (dk, dv))


def test_initial_state_and_scale():
    w = small("osdn-1.3b-apf", B=1, H=2, T=130)
    inp = W.make_inputs(w)
    g = np.random.default_rng(123)
    inp["S0"] = torch.from_numpy(
        g.standard_normal((1, 2, w.Dv, w.Dk)).astype(np.float32) * 0.1)
    inp["d0"] = torch.from_numpy(g.uniform(0.5, 1.5, (1, 2, w.Dk)).astype(np.float32))
    got = gpu_forward(inp, scale=0.25)
    check(got, oracle(inp, scale=0.25), "bf16", "S0,d0,scale")


def test_state_carry_split():
    w = small("osdn-1.3b-apf", B=1, H=2, T=256)
    inp = W.make_inputs(w)
    full = gpu_forward(inp)
    cut = 100   # not a chunk boundary
    a = {k: (v[:, :, :cut].contiguous() if isinstance(v, torch.Tensor) else v)
         for k, v in inp.items()}
    b = {k: (v[:, :, cut:].contiguous() if isinstance(v, torch.Tensor) else v)
         for k, v in inp.items()}
    oa, Sa, da = gpu_forward(a)
    b["S0"] = torch.from_numpy(Sa.astype(np.float32))
    b["d0"] = torch.from_numpy(da.astype(np.float32))
    ob, Sb, db = gpu_forward(b)
    ref = oracle(inp)
    check((np.concatenate([oa, ob], axis=2), Sb, db), ref, "bf16", "split")
    assert rel_l2(np.concatenate([oa, ob], axis=2), full[0]) < 2e-2


def test_in_place_state():
    w = small("osdn-340m", B=1, H=2, T=128)
    inp = W.make_inputs(w)
    x = to_dev(inp)
    S = torch.zeros((1, 2, w.Dv, w.Dk), dtype=torch.float32, device=DEV)
    d = torch.ones((1, 2, w.Dk), dtype=torch.float32, device=DEV)
    o = torch.empty((1, 2, w.T, w.Dv), dtype=torch.bfloat16, device=DEV)
    osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"], None, x["eta"], d, S,
                      chunk=64, out=(o, S, d))
    torch.cuda.synchronize()
    check((W.to_f64(o), W.to_f64(S), W.to_f64(d)), oracle(inp), "bf16",
          "in-place")


def test_beta_zero_leaves_memory():
    w = small("osdn-1.3b-apf", B=1, H=2, T=70)
    inp = W.make_inputs(w)
    inp["beta"] = torch.zeros_like(inp["beta"])
    g = np.random.default_rng(5)
    S0 = g.standard_normal((1, 2, w.Dv, w.Dk)).astype(np.float32)
    inp["S0"] = torch.from_numpy(S0)
    o, S, d = gpu_forward(inp)
    assert np.array_equal(S, S0.astype(np.float64))
    ref = oracle(inp)
    assert rel_l2(o, ref[0]) < 2e-2
    assert rel_l2(d, ref[2]) < D_TOL


def test_empty_sequence_returns_initial_state():
    w = small("osdn-340m", B=2, H=2, T=0)
    inp = W.make_inputs(w)
    g = np.random.default_rng(6)
    inp["S0"] = torch.from_numpy(g.standard_normal((2, 2, w.Dv, w.Dk)).astype(np.float32))
    inp["d0"] = torch.from_numpy(g.uniform(0.5, 2, (2, 2, w.Dk)).astype(np.float32))
    o, S, d = gpu_forward(inp)
    assert o.shape == (2, 2, 0, w.Dv)
    assert np.array_equal(S, W.to_f64(inp["S0"]))
    assert np.array_equal(d, W.to_f64(inp["d0"]))


def test_empty_batch_is_a_no_op():
    w = small("osdn-340m", B=0, H=2, T=64)
    inp = W.make_inputs(w)
    o, S, d = gpu_forward(inp)
    assert o.shape[0] == 0 and S.shape[0] == 0


def test_deltanet_special_case():
    """d0 = 1, eta = 0, no gate: the preconditioner stays 1 exactly and the
    GPU result matches plain DeltaNet."""
    w = small("osdn-340m", B=1, H=2, T=140)
    inp = W.make_inputs(w)
    inp["eta"] = 0.0
    o, S, d = gpu_forward(inp)
    assert np.all(d == 1.0)
    f = W.to_f64
    ro, rS = R.deltanet_ref(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["beta"]))
    assert rel_l2(o, ro) < 2e-2 and rel_l2(S, rS) < 2e-2


def test_precond_scan_alone_and_decoupling():
    w = small("osdn-1.3b-apf", B=2, H=2, T=333)
    inp = W.make_inputs(w)
    x = to_dev(inp)
    kt, dT = osdn.osdn_precond_scan(x["k"], x["beta"], x["r"], x["eta"])
    torch.cuda.synchronize()
    f = W.to_f64
    rkt, rd, _, _ = R.precond_scan_ref(f(inp["k"]), f(inp["beta"]), f(inp["r"]),
                                       inp["eta"])
    assert rel_l2(f(dT), rd) < D_TOL
    assert rel_l2(f(kt), rkt) < 4e-3          # bf16 rounding of k~
    # forward's d_T equals the scan's, bit for bit, whatever q, v and S0 are
    _, _, d1 = gpu_forward(inp)
    inp2 = dict(inp)
    g = torch.Generator().manual_seed(9)
    inp2["q"] = torch.randn(inp["q"].shape, generator=g).to(inp["q"].dtype)
    inp2["v"] = torch.randn(inp["v"].shape, generator=g).to(inp["v"].dtype)
    inp2["S0"] = torch.randn((2, 2, w.Dv, w.Dk), generator=g)
    _, _, d2 = gpu_forward(inp2)
    assert np.array_equal(d1, f(dT)) and np.array_equal(d1, d2)


@pytest.mark.parametrize("chunk", [16, 64])
def test_zero_key_rows(chunk):
    """Tokens whose key is exactly zero (||k||^2 = 0): the gradient step is
    taken as zero there and the write vanishes, in the chunked phase 1 and
    in the engine alike (a zero row inside a chunk, at a chunk's first and
    last position, and a whole zero chunk)."""
    w = small("osdn-1.3b-apf", B=1, H=2, T=64 * 3 + 20)
    inp = W.make_inputs(w)
    k = inp["k"].clone()
    for t in (5, 64, 127, 130):
        k[:, :, t] = 0
    k[:, 1, 128:192] = 0
    inp["k"] = k
    got = gpu_forward(inp, chunk=chunk)
    check(got, oracle(inp), "bf16", "zero keys C=%d" % chunk)


@pytest.mark.parametrize("T,chunk,dtype", [(1, 64, "bf16"), (63, 64, "bf16"),
                                           (64, 64, "bf16"), (65, 64, "bf16"),
                                           (1, 16, "f32"), (17, 16, "f32")])
def test_short_sequences(T, chunk, dtype):
    """Sequences around one chunk: a single token, one token short of a
    chunk, exactly one chunk, one token past it."""
    name = "osdn-1.3b-apf" if dtype == "bf16" else "tiny-fp32"
    w = small(name, B=1, H=2, T=T, chunk=chunk)
    inp = W.make_inputs(w)
    check(gpu_forward(inp), oracle(inp), dtype, "T=%d C=%d" % (T, chunk))


def test_deterministic():
    w = small("osdn-1.3b-apf", B=1, H=4, T=256)
    inp = W.make_inputs(w)
    a, b = gpu_forward(inp), gpu_forward(inp)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# Full workload sizes, in the launch configuration the benchmark times: every
# (batch, head) stream against the oracle at full length, with the
# per-stream and per-token bounds of tests/parity.py beside the tensor one
# (the persistent grids walk several chunks per workgroup only at these
# sizes).
FULL = ["osdn-340m", "osdn-1.3b-apf", "osdn-recall-8k"]


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size_all_streams(name):
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    print("case %s" % name, flush=True)
    o, S, d = gpu_forward(inp)
    ro, rS, rd = oracle(inp)
    check_full(name, w.dtype, o, ro, S, rS, d, rd)


@pytest.mark.parametrize("dk,dv", [(32, 32), (32, 64), (32, 128), (64, 32),
                                   (64, 64), (64, 128)])
def test_fp32_chunk64(dk, dv):
    """The fp32 OSDN forward at chunk 64 (phase 2 forms K~ from the phase-1
    records) for every (Dk, Dv) it supports, with and without the forgetting
    gate, several chunks and a ragged tail."""
    assert osdn.supported(dk, dv, 64, torch.float32)
    for apf in (False, True):
        w = small("osdn-1.3b-apf", B=2, H=2, T=64 * 3 + 21, Dk=dk, Dv=dv,
                  chunk=64, dtype="f32", apf=apf)
        inp = W.make_inputs(w)
        check(gpu_forward(inp), oracle(inp), "f32",
              "fp32 C=64 dk=%d dv=%d apf=%d" % (dk, dv, apf))


def test_fp32_chunk64_many_chunks_per_workgroup():
    """fp32 at chunk 64 with more chunks than the persistent grids have
    workgroups (768 chunks), so every workgroup walks several of them."""
    w = small("osdn-1.3b-apf", B=4, H=32, T=64 * 5 + 3, Dk=64, Dv=64,
              chunk=64, dtype="f32")
    inp = W.make_inputs(w)
    o, S, d = gpu_forward(inp)
    ro, rS, rd = oracle(inp)
    check_full("fp32 C=64 768 chunks", "f32", o, ro, S, rS, d, rd)


def test_nan_stream_is_isolated():
    """A NaN in one (batch, head) stream's value stays in that stream: every
    other stream's o, S_T and d_T are bit-for-bit those of the clean run (the
    NaN in a key reaches d as well, in its own stream only)."""
    w = small("osdn-1.3b-apf", B=2, H=3, T=64 * 4 + 11)
    inp = W.make_inputs(w)
    clean = gpu_forward(inp)
    for key, where in (("v", (1, 2, 70, 5)), ("k", (0, 1, 130, 17)),
                       ("q", (1, 0, 3, 9))):
        bad = dict(inp)
        t = inp[key].clone()
        t[where] = float("nan")
        bad[key] = t
        got = gpu_forward(bad)
        b, h = where[0], where[1]
        for x, y in zip(got, clean):
            mask = np.ones(x.shape[:2], dtype=bool)
            mask[b, h] = False
            assert np.array_equal(x[mask], y[mask]), key
        assert not np.all(np.isfinite(got[0][b, h])), key


# Residual contraction ratios rho_t = (1 - beta_t c_t)^2 and their geometric
# mean per stream. They come from the same fp32 phase-1 arithmetic as d_T, so
# they are held to d_T's bound: relative L2 <= 1e-5 over the compared tensor.
RHO_TOL = 1e-5


def check_rho(rho, qg, inp, where, sl=(slice(None), slice(None))):
    f = lambda key: None if inp.get(key) is None else W.to_f64(inp[key])[sl]
    rr, rq = R.residual_ratio_ref(f("k"), f("beta"), f("r"), inp["eta"], f("d0"))
    er, eq = rel_l2(W.to_f64(rho)[sl], rr), rel_l2(W.to_f64(qg)[sl], rq)
    print("%s: rel_l2 rho=%.3e q_geo=%.3e" % (where, er, eq), flush=True)
    assert er <= RHO_TOL and eq <= RHO_TOL


@pytest.mark.parametrize("w", SMALL, ids=["%s-T%d" % (w.name, w.T) for w in SMALL])
def test_residual_ratio_small(w):
    x = to_dev(W.make_inputs(w))
    inp = W.make_inputs(w)
    o, S, d, rho, qg = osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"],
                                         x["r"], x["eta"], chunk=w.chunk,
                                         diagnostics=True)
    torch.cuda.synchronize()
    check_rho(rho, qg, inp, w.name)
    # asking for the diagnostics changes nothing else
    check((W.to_f64(o), W.to_f64(S), W.to_f64(d)), oracle(inp), w.dtype,
          w.name + " with diagnostics")


def test_residual_ratio_degenerate_steps():
    """Tokens where the step size e_t = eta beta_t / n_t is zero (zero keys,
    beta = 0) take the ratio from the entry preconditioner; eta = 0 makes
    every token do so."""
    w = small("osdn-1.3b-apf", B=1, H=2, T=64 * 2 + 30)
    inp = W.make_inputs(w)
    k = inp["k"].clone()
    k[:, :, 3] = 0
    k[:, 1, 70:80] = 0
    inp["k"] = k
    b = inp["beta"].clone()
    b[:, :, 10] = 0
    b[:, 0, 100:130] = 0
    inp["beta"] = b
    g = np.random.default_rng(8)
    inp["d0"] = torch.from_numpy(g.uniform(0.5, 1.5, (1, 2, w.Dk)).astype(np.float32))
    for eta in (0.1, 0.0):
        inp["eta"] = eta
        x = to_dev(inp)
        _, _, rho, qg = osdn.osdn_precond_scan(x["k"], x["beta"], x["r"], eta,
                                               x["d0"], want_ktilde=False,
                                               diagnostics=True)
        torch.cuda.synchronize()
        check_rho(rho, qg, inp, "degenerate eta=%g" % eta)
        assert np.all(W.to_f64(rho)[0, :, 3] == 1.0)


def test_residual_ratio_chunk16_path_and_empty():
    w = small("osdn-340m", B=2, H=1, T=200, chunk=16)
    inp = W.make_inputs(w)
    x = to_dev(inp)
    _, _, _, rho, qg = osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"],
                                         None, x["eta"], chunk=16,
                                         diagnostics=True)
    torch.cuda.synchronize()
    check_rho(rho, qg, inp, "chunk 16")
    w0 = small("osdn-340m", B=2, H=1, T=0)
    x0 = to_dev(W.make_inputs(w0))
    _, _, _, rho0, qg0 = osdn.osdn_forward(x0["q"], x0["k"], x0["v"],
                                           x0["beta"], None, 0.1,
                                           diagnostics=True)
    torch.cuda.synchronize()
    assert rho0.shape == (2, 1, 0) and torch.all(qg0.cpu() == 1.0)


@pytest.mark.parametrize("name", ["osdn-340m", "osdn-1.3b-apf"])
def test_residual_ratio_full_size_all_streams(name):
    w = W.BY_NAME[name]
    inp = W.make_inputs(w)
    x = to_dev(inp)
    _, _, _, rho, qg = osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"],
                                         x["r"], x["eta"], chunk=w.chunk,
                                         diagnostics=True)
    torch.cuda.synchronize()
    check_rho(rho, qg, inp, name)
    f = lambda key: None if inp.get(key) is None else W.to_f64(inp[key])
    rr, _ = R.residual_ratio_ref(f("k"), f("beta"), f("r"), inp["eta"])
    # per token, absolute (rho is a ratio of losses, (1 - beta c)^2; where
    # beta c is close to 1 a relative measure would divide by ~0)
    err = np.abs(W.to_f64(rho) - rr)
    print("%s: worst token rho abs error %.3e" % (name, err.max()))
    assert err.max() <= 1e-4


def test_forgetting_gate_zero_and_one():
    """Gate values of exactly 0 (full forgetting of the preconditioner) and
    exactly 1 inside chunks, at a chunk's first and last token and for a
    whole chunk: the chunked phase 1 takes log r with r clamped to 1e-30, a
    relative difference the tolerances cannot see."""
    w = small("osdn-1.3b-apf", B=1, H=2, T=64 * 3 + 10)
    inp = W.make_inputs(w)
    r = inp["r"].clone()
    for t in (0, 7, 63, 64, 100):
        r[:, 0, t] = 0.0
    r[:, 1, 128:192] = 0.0
    r[:, 0, 30:50] = 1.0
    inp["r"] = r
    for chunk in (64, 16):
        check(gpu_forward(inp, chunk=chunk), oracle(inp), "bf16",
              "r in {0, 1} C=%d" % chunk)
