"""Out-of-bounds writes, caught without a fault. Every tensor handed to an
entry point is a view into the middle of an allocation of its own: the
inputs, the outputs and the workspace, which is sized exactly as the
library's query reports. A 64 KiB guard region holding a byte pattern lies
on each side of the view. After the call:
* both guards of every buffer still hold the pattern;
* every input holds its values bit for bit;
* every output equals, bit for bit, the output of the same call on
  ordinary buffers (the kernels are deterministic).

The shapes are ragged: several streams and a partial last chunk (T = 150
at chunk 64: chunks of 64, 64 and 22 tokens). Reads beyond a buffer are not
seen here; writes that land within 64 KiB of one are."""
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 1 << 16
PAT = 0xA5
NAN = float("nan")


def _bits(t):
    """The tensor's bytes as integers, for bitwise comparison (NaN-safe)."""
    return t.contiguous().view(torch.uint8)


class Arena:
    """Guarded copies of tensors; check() verifies guards and inputs."""

    def __init__(self):
        self.bufs = []

    def _new(self, nbytes):
        base = torch.full((nbytes + 2 * GUARD,), PAT, dtype=torch.uint8,
                          device=DEV)
        return base, base[GUARD:GUARD + nbytes]

    def inp(self, t):
        """A guarded copy of input t (None stays None)."""
        if not isinstance(t, torch.Tensor):
            return t
        base, mid = self._new(t.numel() * t.element_size())
        v = mid.view(t.dtype).view(t.shape)
        v.copy_(t)
        self.bufs.append((base, v, t.clone()))
        return v

    def out(self, like):
        """A guarded output buffer of like's shape and dtype, NaN-filled."""
        if like is None:
            return None
        base, mid = self._new(like.numel() * like.element_size())
        v = mid.view(like.dtype).view(like.shape)
        v.fill_(NAN)
        self.bufs.append((base, v, None))
        return v

    def workspace(self, nbytes):
        base, mid = self._new(max(int(nbytes), 1))
        self.bufs.append((base, mid, None))
        return mid

    def check(self):
        torch.cuda.synchronize()
        for i, (base, v, orig) in enumerate(self.bufs):
            assert bool((base[:GUARD] == PAT).all()), "guard before buffer %d" % i
            assert bool((base[-GUARD:] == PAT).all()), "guard after buffer %d" % i
            if orig is not None:
                assert torch.equal(_bits(v), _bits(orig)), "input %d changed" % i


def _same(got, ref):
    if isinstance(ref, dict):
        assert set(got) == set(ref)
        for n in ref:
            _same(got[n], ref[n])
        return
    if isinstance(ref, (tuple, list)):
        for a, b in zip(got, ref):
            _same(a, b)
        return
    if ref is None:
        assert got is None
        return
    assert torch.equal(_bits(got), _bits(ref))


def _inputs(name, **scale):
    w = W.BY_NAME[name].scaled(**scale)
    x = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
         for k, v in W.make_inputs(w).items()}
    return w, x


def _code(w):
    return 1 if w.dtype == "bf16" else 0


OSDN_CASES = [
    dict(name="osdn-1.3b-apf", B=2, H=3, T=150),                 # fused, bf16
    dict(name="osdn-1.3b-apf", B=2, H=3, T=150, chunk=32),       # K~ kernel
    dict(name="tiny-fp32", B=2, H=3, T=150, Dk=64, Dv=64, chunk=64),
]


@pytest.mark.parametrize("case", OSDN_CASES, ids=lambda c: "-".join(
    "%s%s" % (k, v) for k, v in c.items()))
def test_guard_osdn_forward(case):
    case = dict(case)
    w, x = _inputs(case.pop("name"), **case)
    print("case:", w, flush=True)
    L = osdn.load_library()
    args = (x["q"], x["k"], x["v"], x["beta"])
    kw = dict(r=x["r"], eta=x["eta"], d0=x["d0"], S0=x["S0"], chunk=w.chunk)
    ref = osdn.osdn_forward(*args, **kw)
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    gkw = {k: a.inp(v) for k, v in kw.items()}
    out = tuple(a.out(t) for t in ref)
    ws = a.workspace(L.osdn_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                                    w.chunk, _code(w)))
    got = osdn.osdn_forward(*gargs, **gkw, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_phase1_and_phase2_alone():
    w, x = _inputs("osdn-1.3b-apf", B=2, H=3, T=150, chunk=32)
    print("case:", w, flush=True)
    L = osdn.load_library()
    kt, dT = osdn.osdn_precond_scan(x["k"], x["beta"], r=x["r"], eta=x["eta"])
    a = Arena()
    gk, gb, gr = a.inp(x["k"]), a.inp(x["beta"]), a.inp(x["r"])
    out = (a.out(kt), a.out(dT))
    ws = a.workspace(L.osdn_precond_workspace_bytes(w.B, w.H, w.T, w.Dk,
                                                    _code(w)))
    got = osdn.osdn_precond_scan(gk, gb, r=gr, eta=x["eta"], out=out,
                                 workspace=ws)
    a.check()
    _same(got, (kt, dT))

    ref = osdn.osdn_chunk_forward(x["q"], x["k"], kt, x["v"], x["beta"],
                                  chunk=w.chunk)
    a = Arena()
    gargs = tuple(a.inp(t) for t in (x["q"], x["k"], kt, x["v"], x["beta"]))
    out = tuple(a.out(t) for t in ref)
    ws = a.workspace(L.osdn_chunk_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                                  w.chunk, _code(w)))
    got = osdn.osdn_chunk_forward(*gargs, chunk=w.chunk, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_gdn2_forward():
    w, x = _inputs("gdn2-1.3b", B=2, H=3, T=150)
    print("case:", w, flush=True)
    L = osdn.load_library()
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"])
    ref = osdn.gdn2_forward(*args, chunk=w.chunk)
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    out = tuple(a.out(t) for t in ref)
    ws = a.workspace(L.gdn2_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                                    w.chunk, _code(w)))
    got = osdn.gdn2_forward(*gargs, chunk=w.chunk, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_osdn_gated_forward():
    w, x = _inputs("osdn-gated-1.3b", B=2, H=3, T=150)
    print("case:", w, flush=True)
    L = osdn.load_library()
    args = (x["q"], x["k"], x["v"], x["beta"], x["log_alpha"])
    kw = dict(r=x["r"], eta=x["eta"], chunk=w.chunk)
    ref = osdn.osdn_gated_forward(*args, **kw)
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    gkw = {k: a.inp(v) for k, v in kw.items()}
    out = tuple(a.out(t) for t in ref)
    ws = a.workspace(L.osdn_gated_forward_workspace_bytes(
        w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, _code(w)))
    got = osdn.osdn_gated_forward(*gargs, **gkw, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_decode():
    """The recurrent decodes update the state in place: the guarded state
    buffers are compared with a plain call's, as outputs."""
    w, x = _inputs("osdn-decode", B=3, H=5, T=3)
    print("case:", w, flush=True)
    S, d = x["S0"].clone(), x["d0"].clone()
    o = osdn.osdn_decode(x["q"], x["k"], x["v"], x["beta"], S, d, r=x["r"],
                         eta=x["eta"])
    a = Arena()
    gq, gk, gv, gb, gr = (a.inp(x[n]) for n in ("q", "k", "v", "beta", "r"))
    gS, gd = a.out(S), a.out(d)
    gS.copy_(x["S0"])
    gd.copy_(x["d0"])
    go = a.out(o)
    got = osdn.osdn_decode(gq, gk, gv, gb, gS, gd, r=gr, eta=x["eta"], out=go)
    a.check()
    _same((got, gS, gd), (o, S, d))

    w, x = _inputs("gdn2-decode", B=3, H=5, T=3)
    print("case:", w, flush=True)
    S = x["S0"].clone()
    args = [x[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o = osdn.gdn2_decode(*args, S)
    a = Arena()
    gargs = [a.inp(t) for t in args]
    gS = a.out(S)
    gS.copy_(x["S0"])
    go = a.out(o)
    got = osdn.gdn2_decode(*gargs, gS, out=go)
    a.check()
    _same((got, gS), (o, S))


def _cot(w):
    c = W.make_cotangents(w)
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in c.items()}


def test_guard_osdn_backward():
    w, x = _inputs("osdn-1.3b-apf", B=2, H=3, T=150)
    print("case:", w, flush=True)
    L = osdn.load_library()
    c = _cot(w)
    args = (x["q"], x["k"], x["v"], x["beta"], c["do"])
    kw = dict(r=x["r"], eta=x["eta"], dS_T=c["dS_T"], dd_T=c["dd_T"])
    ref = osdn.osdn_backward(*args, **kw)
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    gkw = {k: a.inp(v) for k, v in kw.items()}
    out = {n: a.out(t) for n, t in ref.items()}
    ws = a.workspace(L.osdn_backward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv))
    got = osdn.osdn_backward(*gargs, **gkw, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_gated_backwards():
    w, x = _inputs("osdn-gated-1.3b", B=2, H=3, T=150)
    print("case:", w, flush=True)
    L = osdn.load_library()
    c = _cot(w)
    args = (x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], c["do"])
    kw = dict(r=x["r"], eta=x["eta"], dS_T=c["dS_T"], dd_T=c["dd_T"])
    ref = osdn.osdn_gated_backward(*args, **kw)
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    gkw = {k: a.inp(v) for k, v in kw.items()}
    out = {n: a.out(t) for n, t in ref.items()}
    ws = a.workspace(L.osdn_gated_backward_workspace_bytes(w.B, w.H, w.T, w.Dk,
                                                           w.Dv))
    got = osdn.osdn_gated_backward(*gargs, **gkw, out=out, workspace=ws)
    a.check()
    _same(got, ref)

    w, x = _inputs("gdn2-1.3b", B=2, H=3, T=150)
    print("case:", w, flush=True)
    c = _cot(w)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], c["do"])
    ref = osdn.gdn2_backward(*args, dS_T=c["dS_T"])
    a = Arena()
    gargs = tuple(a.inp(t) for t in args)
    gdS = a.inp(c["dS_T"])
    out = {n: a.out(t) for n, t in ref.items()}
    ws = a.workspace(L.gdn2_backward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv))
    got = osdn.gdn2_backward(*gargs, dS_T=gdS, out=out, workspace=ws)
    a.check()
    _same(got, ref)


def test_guard_check_sees_a_write_into_a_guard():
    """The checker itself: a byte written into a guard region (by torch,
    inside the allocation) and a changed input are both reported."""
    a = Arena()
    t = a.inp(torch.ones(100, device=DEV))
    a.check()
    a.bufs[0][0][GUARD + t.numel() * 4 + 7] = 0  # just past the view
    with pytest.raises(AssertionError, match="guard after"):
        a.check()
    a = Arena()
    t = a.inp(torch.ones(100, device=DEV))
    t[3] = 2.0
    with pytest.raises(AssertionError, match="input 0 changed"):
        a.check()
