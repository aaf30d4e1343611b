"""The seeded input generators: shapes, dtypes, determinism, distributions."""
import numpy as np
import pytest
import torch

import workloads as W


@pytest.mark.parametrize("w", W.WORKLOADS, ids=[w.name for w in W.WORKLOADS])
def test_shapes_and_dtypes_small(w):
    ws = w.scaled(B=1, H=2, T=2 * w.chunk)
    x = W.make_inputs(ws)
    dt = W.torch_dtype(w.dtype)
    assert x["q"].shape == (1, 2, ws.T, w.Dk) and x["q"].dtype == dt
    assert x["k"].shape == (1, 2, ws.T, w.Dk) and x["k"].dtype == dt
    assert x["v"].shape == (1, 2, ws.T, w.Dv) and x["v"].dtype == dt
    if w.kind == "osdn":
        assert x["beta"].shape == (1, 2, ws.T) and x["beta"].dtype == torch.float32
        assert (x["r"] is not None) == w.apf
        b = x["beta"].double()
        assert torch.all((b > 0) & (b < 1))
        if w.decay:
            assert x["log_alpha"].shape == (1, 2, ws.T, w.Dk)
            assert torch.all(x["log_alpha"] < 0)
        else:
            assert "log_alpha" not in x
    else:
        assert x["log_alpha"].shape == (1, 2, ws.T, w.Dk)
        assert torch.all(x["log_alpha"] < 0)
        assert x["b"].shape == (1, 2, ws.T, w.Dk) and x["b"].dtype == dt
        assert x["w"].shape == (1, 2, ws.T, w.Dv) and x["w"].dtype == dt
    if w.state:
        Ssh = (1, 2, w.Dv, w.Dk) if w.kind == "osdn" else (1, 2, w.Dk, w.Dv)
        assert x["S0"].shape == Ssh and x["S0"].dtype == torch.float32
        if w.kind == "osdn":
            d0 = x["d0"].double()
            assert d0.shape == (1, 2, w.Dk)
            assert torch.all((d0 >= 0.5) & (d0 <= 1.5))
    else:
        assert x["S0"] is None
    n = x["k"].double().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=2e-2)


def test_deterministic():
    w = W.BY_NAME["osdn-1.3b-apf"].scaled(B=1, H=2, T=128)
    a, b = W.make_inputs(w), W.make_inputs(w)
    for key in ("q", "k", "v", "beta", "r"):
        assert torch.equal(a[key], b[key])


def test_recall_queries_repeat_earlier_keys():
    w = W.BY_NAME["osdn-recall-8k"].scaled(B=1, H=2, T=256)
    x = W.make_inputs(w)
    k, q = x["k"], x["q"]
    for t in range(1, 256, 17):
        hits = (k[0, 0, :t] == q[0, 0, t]).all(dim=-1)
        assert hits.any()
    assert torch.equal(q[0, 0, 0], k[0, 0, 0])
    # pool keys repeat: far fewer distinct keys than tokens
    distinct = torch.unique(k[0, 0].view(torch.int16), dim=0).shape[0]
    assert distinct < 256
