"""The forward and backward entry points under HIP graph capture: every
kernel launch of a call goes into the graph (the library issues no memsets and allocates
nothing), and each replay, with other eager work and synchronisations in
between, reproduces the eager result bit for bit (the kernels are
deterministic)."""
import pytest
import torch

import delta_rule_recurrent_scan_amd as osdn
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
            for k, v in inp.items()}


def _replay_matches(run, outs, n_replays=3):
    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(n_replays):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), "replay %d differs from the eager call" % i


def test_osdn_forward_graph_replay():
    w = W.BY_NAME["osdn-1.3b-apf"].scaled(B=2, H=4, T=64 * 5 + 13)
    x = _dev(W.make_inputs(w))
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((w.B, w.H, w.Dv, w.Dk), dtype=torch.float32, device=DEV)
    d = torch.empty((w.B, w.H, w.Dk), dtype=torch.float32, device=DEV)
    need = osdn.workspace_bytes(w.B, w.H, w.T, w.Dk, w.Dv, 64, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def run():
        return osdn.osdn_forward(x["q"], x["k"], x["v"], x["beta"], x["r"],
                                 x["eta"], out=(o, S, d), workspace=ws)
    _replay_matches(run, [o, S, d])


def test_gdn2_forward_graph_replay():
    w = W.BY_NAME["gdn2-1.3b"].scaled(B=1, H=4, T=64 * 3 + 7)
    x = _dev(W.make_inputs(w))
    o = torch.empty((w.B, w.H, w.T, w.Dv), dtype=torch.bfloat16, device=DEV)
    S = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=DEV)
    need = osdn.load_library().gdn2_forward_workspace_bytes(
        w.B, w.H, w.T, w.Dk, w.Dv, 64, 1)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)

    def run():
        return osdn.gdn2_forward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                                 x["w"], out=(o, S), workspace=ws)
    _replay_matches(run, [o, S])


def _grad_outs(shapes):
    return {n: torch.empty(s, dtype=torch.float32, device=DEV)
            for n, s in shapes.items()}


def test_osdn_backward_graph_replay():
    w = W.BY_NAME["osdn-1.3b-apf"].scaled(B=1, H=4, T=64 * 3 + 5)
    x = _dev(W.make_inputs(w))
    c = _dev(W.make_cotangents(w))
    B, H, T, Dk, Dv = w.B, w.H, w.T, w.Dk, w.Dv
    g = _grad_outs(dict(q=(B, H, T, Dk), k=(B, H, T, Dk), v=(B, H, T, Dv),
                        beta=(B, H, T), r=(B, H, T), eta=(B, H),
                        d0=(B, H, Dk), S0=(B, H, Dv, Dk)))
    ws = torch.empty(osdn.backward_workspace_bytes(B, H, T, Dk, Dv),
                     dtype=torch.uint8, device=DEV)

    def run():
        osdn.osdn_backward(x["q"], x["k"], x["v"], x["beta"], c["do"],
                           r=x["r"], eta=x["eta"], dS_T=c["dS_T"],
                           dd_T=c["dd_T"], out=g, workspace=ws)
        return list(g.values())
    _replay_matches(run, list(g.values()))


@pytest.mark.parametrize("kind", ["gdn2", "gated"])
def test_gate_aware_backward_graph_replay(kind):
    base = "gdn2-1.3b" if kind == "gdn2" else "osdn-gated-1.3b"
    w = W.BY_NAME[base].scaled(B=1, H=2, T=64 * 2 + 9, state=True)
    x = _dev(W.make_inputs(w))
    c = _dev(W.make_cotangents(w))
    B, H, T, Dk, Dv = w.B, w.H, w.T, w.Dk, w.Dv
    if kind == "gdn2":
        g = _grad_outs(dict(q=(B, H, T, Dk), k=(B, H, T, Dk), v=(B, H, T, Dv),
                            log_alpha=(B, H, T, Dk), b=(B, H, T, Dk),
                            w=(B, H, T, Dv), S0=(B, H, Dk, Dv)))
        ws = torch.empty(osdn.gdn2_backward_workspace_bytes(B, H, T, Dk, Dv),
                         dtype=torch.uint8, device=DEV)

        def run():
            osdn.gdn2_backward(x["q"], x["k"], x["v"], x["log_alpha"], x["b"],
                               x["w"], c["do"], S0=x["S0"], dS_T=c["dS_T"],
                               out=g, workspace=ws)
            return list(g.values())
    else:
        g = _grad_outs(dict(q=(B, H, T, Dk), k=(B, H, T, Dk), v=(B, H, T, Dv),
                            beta=(B, H, T), r=(B, H, T), eta=(B, H),
                            log_alpha=(B, H, T, Dk), d0=(B, H, Dk),
                            S0=(B, H, Dv, Dk)))
        ws = torch.empty(osdn.gated_backward_workspace_bytes(B, H, T, Dk, Dv),
                         dtype=torch.uint8, device=DEV)

        def run():
            osdn.osdn_gated_backward(
                x["q"], x["k"], x["v"], x["beta"], x["log_alpha"], c["do"],
                r=x["r"], eta=x["eta"], d0=x["d0"], S0=x["S0"],
                dS_T=c["dS_T"], dd_T=c["dd_T"], out=g, workspace=ws)
            return list(g.values())
    _replay_matches(run, list(g.values()))
