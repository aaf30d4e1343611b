"""The forward entry points under HIP graph capture: every kernel launch of a
call goes into the graph (the library issues no memsets and allocates
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
