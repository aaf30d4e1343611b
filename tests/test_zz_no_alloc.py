"""GPU check of osdn_forward_noalloc (the forward on the library's static
per-device scratch) against osdn_forward with a caller workspace, through the
C ABI: two calls in a row, the second on a smaller input, each bit for bit
equal to the workspace call (the same kernels run on the same inputs)."""
import ctypes

import numpy as np
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _call(L, fn, w, x, with_ws):
    P = osdn._ptr
    code = 1 if w.dtype == "bf16" else 0
    dt = W.torch_dtype(w.dtype)
    o = torch.full((w.B, w.H, w.T, w.Dv), float("nan"), dtype=dt, device=DEV)
    S = torch.full((w.B, w.H, w.Dv, w.Dk), float("nan"), device=DEV)
    d = torch.full((w.B, w.H, w.Dk), float("nan"), device=DEV)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [w.B, w.H, w.T, w.Dk, w.Dv, w.chunk, code, P(x["q"]), P(x["k"]),
            P(x["v"]), P(x["beta"]), P(x["r"]), float(w.eta), None, None, 1.0,
            P(o), P(S), P(d), None, None]
    if with_ws:
        n = L.osdn_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, w.chunk,
                                           code)
        ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV)
        rc = fn(*args, P(ws), ws.numel(), sp)
    else:
        rc = fn(*args, sp)
    assert rc == 0, L.osdn_strerror(rc)
    torch.cuda.synchronize()
    return [W.to_f64(t) for t in (o, S, d)]


def test_noalloc_matches_workspace_forward_twice():
    L = osdn.load_library()
    base = W.BY_NAME["osdn-1.3b-apf"]
    for i, w in enumerate([base.scaled(B=2, H=8, T=1500),
                           base.scaled(B=1, H=3, T=333)]):
        need = L.osdn_forward_workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv,
                                              w.chunk, 1)
        assert need <= osdn.NOALLOC_SCRATCH_BYTES
        print("call %d: %s, scratch %d bytes" % (i, w, need), flush=True)
        x = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
             for k, v in W.make_inputs(w).items()}
        got = _call(L, L.osdn_forward_noalloc, w, x, False)
        ref = _call(L, L.osdn_forward, w, x, True)
        for a, b in zip(got, ref):
            assert np.all(np.isfinite(a))
            assert np.array_equal(a, b)
