"""Seeded synthetic inputs for the OSDN and GDN-2 forward passes.

This module holds input generation only: random draws, the L2 row
normalisation of q and k and the rounding to the storage dtype. It contains
none of the method's arithmetic. Both the CPU oracle (through the tests) and
the HIP path consume exactly the tensors produced here, so bf16 inputs reach
the oracle as the same bits, widened to float64.

Workloads (dims B, H, T, Dk, Dv and chunk C):

1. tiny fp32 OSDN: 1, 2, 256, 32, 32, C=16; eta 0.1; no forgetting gate.
2. 340M-layer shape: 8, 8, 2048, 128, 128, C=64; bf16 q/k/v; no gate.
3. 1.3B-layer shape: 4, 16, 4096, 128, 128, C=64; bf16; forgetting gate
   r = sigmoid(N(2, 0.5)) per token and head.
4. long-context multi-key recall shape: 2, 16, 8192, 128, 128, C=64; keys
   from a per-head pool of 512 unit vectors with 20 % fresh keys; queries
   repeat earlier keys; beta = sigmoid(N(1,1)); gate on; eta 0.05.
5. Gated DeltaNet-2: 4, 16, 4096, 128, 128, C=64; bf16; per-channel decay
   log alpha = -0.1 softplus(N(0,1)); erase/write gates sigmoid(N(0,1)).
6. OSDN recurrent decode at the 1.3B-layer head shape with a serving batch:
   128, 16, 1, 128, 128; bf16; gate on; a drawn initial state, S0 =
   N(0,1)/sqrt(Dk) and d0 = U(0.5, 1.5).
7. GDN-2 recurrent decode, same shape and gates as 5, S0 = N(0,1)/sqrt(Dk).
8. OSDN on a per-channel-decay backbone at the 1.3B-layer shape: as 3, plus
   log alpha = -0.1 softplus(N(0,1)) per key channel (the decay of 5).

Seeds: workload i draws from numpy SeedSequence(i - 1); each tensor comes
from its own spawned child, in the fixed order q, k, v, beta, r, alpha, b, w,
S0, d0.
"""

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "osdn" or "gdn2"
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str           # "f32" or "bf16": storage dtype of q, k, v (b, w), o
    eta: float = 0.1
    apf: bool = False    # forgetting gate r present
    beta_mu: float = 0.0  # beta = sigmoid(N(beta_mu, 1))
    keys: str = "gauss"  # "gauss" or "pool" (multi-key recall)
    seed: int = 0
    state: bool = False  # draw an initial state S0 (and d0 for OSDN)
    decay: bool = False  # OSDN on a decaying backbone: log alpha per channel

    @property
    def tokens(self):
        return self.B * self.T

    def scaled(self, **kw):
        """Same recipe at other sizes (for oracle-sized parity cases)."""
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny-fp32", "osdn", 1, 2, 256, 32, 32, 16, "f32", seed=0),
    Workload("osdn-340m", "osdn", 8, 8, 2048, 128, 128, 64, "bf16", seed=1),
    Workload("osdn-1.3b-apf", "osdn", 4, 16, 4096, 128, 128, 64, "bf16",
             apf=True, seed=2),
    Workload("osdn-recall-8k", "osdn", 2, 16, 8192, 128, 128, 64, "bf16",
             eta=0.05, apf=True, beta_mu=1.0, keys="pool", seed=3),
    Workload("gdn2-1.3b", "gdn2", 4, 16, 4096, 128, 128, 64, "bf16", seed=4),
    Workload("osdn-decode", "osdn", 128, 16, 1, 128, 128, 64, "bf16",
             apf=True, seed=5, state=True),
    Workload("gdn2-decode", "gdn2", 128, 16, 1, 128, 128, 64, "bf16", seed=6,
             state=True),
    Workload("osdn-gated-1.3b", "osdn", 4, 16, 4096, 128, 128, 64, "bf16",
             apf=True, seed=7, decay=True),
]

BY_NAME = {w.name: w for w in WORKLOADS}

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _TORCH_DTYPE[name]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _unit_rows(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return x / np.where(n > 0.0, n, 1.0)


def _store(x, dtype):
    """float64 -> float32 -> storage dtype (bf16 by round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_TORCH_DTYPE[dtype]).contiguous()


def _pool_keys(rng, B, H, T, Dk):
    """Keys from a per-head pool of 512 unit vectors, 20 % fresh unit keys.

    Returns k as a float64 array [B, H, T, Dk].
    """
    pool = _unit_rows(rng.standard_normal((H, 512, Dk)))
    pick = rng.integers(0, 512, size=(B, H, T))
    fresh = rng.random((B, H, T)) < 0.2
    k = pool[np.arange(H)[None, :, None], pick]
    k_new = _unit_rows(rng.standard_normal((B, H, T, Dk)))
    k = np.where(fresh[..., None], k_new, k)
    return k


def _pool_queries(rng, k_stored):
    """q_t is a bit copy of k_s, s uniform over earlier tokens; q_1 = k_1."""
    B, H, T, _ = k_stored.shape
    t = np.arange(T)
    src = np.floor(rng.random((B, H, T)) * np.maximum(t, 1)).astype(np.int64)
    src[..., 0] = 0
    src = np.minimum(src, np.maximum(t - 1, 0))
    idx = torch.from_numpy(src)[..., None].expand(B, H, T, k_stored.shape[-1])
    return torch.gather(k_stored, 2, idx).contiguous()


def make_inputs(w: Workload):
    """Generate one workload's inputs as CPU torch tensors.

    OSDN: dict(q, k, v, beta, r, eta, d0, S0, chunk).
    GDN-2: dict(q, k, v, log_alpha, b, w, S0, chunk).
    S0 and d0 are None (zeros, ones) unless the workload draws a state.
    """
    ss = np.random.SeedSequence(w.seed)
    ch = [np.random.default_rng(s) for s in ss.spawn(10)]
    B, H, T, Dk, Dv = w.B, w.H, w.T, w.Dk, w.Dv
    if w.keys == "pool":
        k = _store(_pool_keys(ch[1], B, H, T, Dk), w.dtype)
        q = _pool_queries(ch[0], k)
    else:
        q = _store(_unit_rows(ch[0].standard_normal((B, H, T, Dk))), w.dtype)
        k = _store(_unit_rows(ch[1].standard_normal((B, H, T, Dk))), w.dtype)
    v = _store(ch[2].standard_normal((B, H, T, Dv)), w.dtype)
    out = dict(q=q, k=k, v=v, chunk=w.chunk, S0=None)
    if w.kind == "osdn":
        beta = _store(_sigmoid(ch[3].standard_normal((B, H, T)) + w.beta_mu),
                      "f32")
        r = (_store(_sigmoid(ch[4].normal(2.0, 0.5, (B, H, T))), "f32")
             if w.apf else None)
        out.update(beta=beta, r=r, eta=w.eta, d0=None)
        if w.decay:
            la = -0.1 * _softplus(ch[5].standard_normal((B, H, T, Dk)))
            out["log_alpha"] = _store(la, "f32")
        if w.state:
            out["S0"] = _store(ch[8].standard_normal((B, H, Dv, Dk))
                               / np.sqrt(Dk), "f32")
            out["d0"] = _store(ch[9].uniform(0.5, 1.5, (B, H, Dk)), "f32")
    else:
        la = -0.1 * _softplus(ch[5].standard_normal((B, H, T, Dk)))
        out.update(log_alpha=_store(la, "f32"),
                   b=_store(_sigmoid(ch[6].standard_normal((B, H, T, Dk))),
                            w.dtype),
                   w=_store(_sigmoid(ch[7].standard_normal((B, H, T, Dv))),
                            w.dtype))
        if w.state:
            out["S0"] = _store(ch[8].standard_normal((B, H, Dk, Dv))
                               / np.sqrt(Dk), "f32")
    return out


def make_cotangents(w: Workload, state=True):
    """Seeded adjoints of the outputs for backward tests: dict(do, dS_T,
    dd_T) as CPU tensors. do [B,H,T,Dv] ~ N(0,1) in the storage dtype; with
    ``state``, dS_T ~ N(0,1)/sqrt(Dk) in fp32, of the state's shape ([B,H,Dv,
    Dk] for OSDN, [B,H,Dk,Dv] for GDN-2), and for OSDN dd_T [B,H,Dk] ~ N(0,1)
    (else None). Drawn from SeedSequence(seed) children 10-12, after the ten
    of make_inputs."""
    ch = [np.random.default_rng(s)
          for s in np.random.SeedSequence(w.seed).spawn(13)[10:]]
    B, H, T, Dk, Dv = w.B, w.H, w.T, w.Dk, w.Dv
    out = dict(do=_store(ch[0].standard_normal((B, H, T, Dv)), w.dtype),
               dS_T=None, dd_T=None)
    if state:
        shape = (B, H, Dk, Dv) if w.kind == "gdn2" else (B, H, Dv, Dk)
        out["dS_T"] = _store(ch[1].standard_normal(shape) / np.sqrt(Dk), "f32")
        if w.kind != "gdn2":
            out["dd_T"] = _store(ch[2].standard_normal((B, H, Dk)), "f32")
    return out


def to_f64(t):
    """Exact widening of a (possibly bf16) CPU/GPU tensor to float64 NumPy."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
