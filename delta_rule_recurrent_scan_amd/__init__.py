"""Python binding of libosdn.so, the MI355X (gfx950) OSDN / GDN-2 forward library.

Argument marshalling only: shapes and dtypes are checked, outputs and the
workspace are allocated with PyTorch on the inputs' device, and the C ABI
(include/osdn.h) is called with raw device pointers and the current HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback. If the library is missing, every call raises.
"""

import ctypes
import os

import torch

__all__ = ["osdn_forward", "osdn_forward_noalloc", "osdn_backward",
           "osdn_gated_backward", "gdn2_backward", "osdn_precond_scan",
           "osdn_chunk_forward",
           "gdn2_forward", "osdn_gated_forward", "osdn_decode",
           "gdn2_decode",
           "workspace_bytes", "precond_workspace_bytes", "supported",
           "kernel_timing", "kernel_times",
           "OsdnError", "library_path", "load_library"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libosdn.so")
_lib = None

OSDN_F32, OSDN_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: OSDN_F32, torch.bfloat16: OSDN_BF16}


class OsdnError(RuntimeError):
    def __init__(self, status, where):
        msg = load_library().osdn_strerror(status).decode()
        super().__init__("%s failed with status %d: %s" % (where, status, msg))
        self.status = status


def library_path():
    return _LIB_PATH


def load_library():
    """Load libosdn.so (built in-tree); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            "libosdn.so is not built (%s); run "
            "`python -m delta_rule_recurrent_scan_amd.build`" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.osdn_strerror.argtypes = [I]
    L.osdn_strerror.restype = ctypes.c_char_p
    L.osdn_forward_supported.argtypes = [I, I, I, I]
    L.osdn_forward_supported.restype = I
    L.osdn_forward_workspace_bytes.argtypes = [I] * 7
    L.osdn_forward_workspace_bytes.restype = Z
    L.osdn_forward.argtypes = ([I] * 7 + [P, P, P, P, P, F, P, P, F, P, P, P, P,
                                          P, P, Z, P])
    L.osdn_forward.restype = I
    L.osdn_precond_workspace_bytes.argtypes = [I] * 5
    L.osdn_precond_workspace_bytes.restype = Z
    L.osdn_precond_scan.argtypes = [I, I, I, I, I, P, P, P, F, P, P, P, P, P,
                                    P, Z, P]
    L.osdn_precond_scan.restype = I
    L.osdn_chunk_workspace_bytes.argtypes = [I] * 7
    L.osdn_chunk_workspace_bytes.restype = Z
    L.osdn_chunk_forward.argtypes = ([I] * 7 + [P, P, P, P, P, P, F, P, P, P,
                                                Z, P])
    L.osdn_chunk_forward.restype = I
    L.gdn2_forward_supported.argtypes = [I, I, I, I]
    L.gdn2_forward_supported.restype = I
    L.gdn2_forward_workspace_bytes.argtypes = [I] * 7
    L.gdn2_forward_workspace_bytes.restype = Z
    L.gdn2_forward.argtypes = ([I] * 7 + [P, P, P, P, P, P, P, F, P, P, P, Z,
                                          P])
    L.gdn2_forward.restype = I
    L.osdn_decode.argtypes = [I] * 6 + [P, P, P, P, P, F, P, P, P, F, P, P]
    L.osdn_gated_forward_supported.argtypes = [I, I, I, I]
    L.osdn_gated_forward_supported.restype = I
    L.osdn_gated_forward_workspace_bytes.argtypes = [I] * 7
    L.osdn_gated_forward_workspace_bytes.restype = Z
    L.osdn_gated_forward.argtypes = ([I] * 7 + [P, P, P, P, P, F, P, P, P, F, P,
                                                P, P, P, Z, P])
    L.osdn_gated_forward.restype = I
    L.osdn_decode.restype = I
    L.gdn2_decode.argtypes = [I] * 6 + [P, P, P, P, P, P, P, F, P, P]
    L.gdn2_decode.restype = I
    L.osdn_forward_noalloc.argtypes = ([I] * 7 + [P, P, P, P, P, F, P, P, F,
                                                  P, P, P, P, P, P])
    L.osdn_forward_noalloc.restype = I
    L.osdn_backward_workspace_bytes.argtypes = [I] * 5
    L.osdn_backward_workspace_bytes.restype = Z
    L.osdn_backward.argtypes = ([I] * 6 + [P, P, P, P, P, F, P, P, F, P, P, P]
                                + [P] * 8 + [P, Z, P])
    L.osdn_backward.restype = I
    L.osdn_gated_backward_workspace_bytes.argtypes = [I] * 5
    L.osdn_gated_backward_workspace_bytes.restype = Z
    L.osdn_gated_backward.argtypes = ([I] * 6 + [P, P, P, P, P, F, P, P, P, F,
                                                 P, P, P] + [P] * 9 + [P, Z, P])
    L.osdn_gated_backward.restype = I
    L.gdn2_backward_workspace_bytes.argtypes = [I] * 5
    L.gdn2_backward_workspace_bytes.restype = Z
    L.gdn2_backward.argtypes = ([I] * 6 + [P] * 7 + [F, P, P] + [P] * 7
                                + [P, Z, P])
    L.gdn2_backward.restype = I
    L.osdn_kernel_timing.argtypes = [I]
    L.osdn_kernel_timing.restype = None
    L.osdn_kernel_times.argtypes = [I, P, P, P]
    L.osdn_kernel_times.restype = I
    _lib = L
    return L


def kernel_timing(enable):
    """Start (clearing earlier records) or stop per-kernel HIP-event timing
    inside the library."""
    load_library().osdn_kernel_timing(1 if enable else 0)


def kernel_times():
    """{kernel name: (launches, mean ms)} of the kernels launched while
    timing was enabled (waits for their events)."""
    L = load_library()
    n = 16
    names = (ctypes.c_char_p * n)()
    counts = (ctypes.c_int * n)()
    ms = (ctypes.c_float * n)()
    k = L.osdn_kernel_times(n, names, counts, ms)
    if k < 0:
        raise RuntimeError("osdn_kernel_times: HIP runtime error")
    return {names[i].decode(): (counts[i], ms[i]) for i in range(min(k, n))}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape),
                                                           tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def supported(Dk, Dv, chunk, dtype):
    return bool(load_library().osdn_forward_supported(Dk, Dv, chunk,
                                                      _DTYPE_CODE[dtype]))


def workspace_bytes(B, H, T, Dk, Dv, chunk, dtype):
    return int(load_library().osdn_forward_workspace_bytes(
        B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dtype]))


def osdn_forward(q, k, v, beta, r=None, eta=0.1, d0=None, S0=None, chunk=64,
                 scale=1.0, out=None, workspace=None, diagnostics=False):
    """OSDN forward on the GPU: returns (o, S_T, d_T), and with
    ``diagnostics=True`` also (rho [B,H,T], q_geo [B,H]): the per-token
    residual contraction ratios (1 - beta_t <d_t, k_t^2>)^2 and their
    geometric mean per stream.

    q, k: [B,H,T,Dk]; v: [B,H,T,Dv] (fp32 or bf16, one dtype); beta, r:
    [B,H,T] fp32 (r=None: no forgetting gate); d0: [B,H,Dk] fp32 (None: ones);
    S0: [B,H,Dv,Dk] fp32 (None: zeros). ``out`` may pass preallocated
    (o, S_T, d_T) (S_T or d_T may be None to skip it) and ``workspace`` a
    preallocated uint8 device buffer, so that a call allocates nothing.
    """
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(r, "r", (B, H, T), torch.float32, dev)
    _check(d0, "d0", (B, H, Dk), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if out is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
        d_T = torch.empty((B, H, Dk), dtype=torch.float32, device=dev)
    else:
        o, S_T, d_T = out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    _check(S_T, "S_T", (B, H, Dv, Dk), torch.float32, dev)
    _check(d_T, "d_T", (B, H, Dk), torch.float32, dev)
    need = L.osdn_forward_workspace_bytes(B, H, T, Dk, Dv, chunk,
                                          _DTYPE_CODE[dt])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rho = qg = None
    if diagnostics:
        rho = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        qg = torch.empty((B, H), dtype=torch.float32, device=dev)
    rc = L.osdn_forward(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt], _ptr(q),
                        _ptr(k), _ptr(v), _ptr(beta), _ptr(r), float(eta),
                        _ptr(d0), _ptr(S0), float(scale), _ptr(o), _ptr(S_T),
                        _ptr(d_T), _ptr(rho), _ptr(qg), _ptr(workspace),
                        workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_forward")
    if diagnostics:
        return o, S_T, d_T, rho, qg
    return o, S_T, d_T


NOALLOC_SCRATCH_BYTES = 128 << 20  # OSDN_NOALLOC_SCRATCH_BYTES


def osdn_forward_noalloc(q, k, v, beta, r=None, eta=0.1, d0=None, S0=None,
                         chunk=64, scale=1.0, out=None):
    """osdn_forward on the library's static per-device scratch (no workspace
    argument, nothing allocated by the call itself when ``out`` is given):
    returns (o, S_T, d_T). Raises OsdnError (workspace) when the sizes need
    more than NOALLOC_SCRATCH_BYTES of scratch. Calls that overlap in time
    on one device share that scratch and must be ordered by the caller."""
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(r, "r", (B, H, T), torch.float32, dev)
    _check(d0, "d0", (B, H, Dk), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if out is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
        d_T = torch.empty((B, H, Dk), dtype=torch.float32, device=dev)
    else:
        o, S_T, d_T = out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    _check(S_T, "S_T", (B, H, Dv, Dk), torch.float32, dev)
    _check(d_T, "d_T", (B, H, Dk), torch.float32, dev)
    rc = L.osdn_forward_noalloc(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt],
                                _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                                float(eta), _ptr(d0), _ptr(S0), float(scale),
                                _ptr(o), _ptr(S_T), _ptr(d_T), None, None,
                                _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_forward_noalloc")
    return o, S_T, d_T


def backward_workspace_bytes(B, H, T, Dk, Dv):
    return int(load_library().osdn_backward_workspace_bytes(B, H, T, Dk, Dv))


def osdn_backward(q, k, v, beta, dout, r=None, eta=0.1, d0=None, S0=None,
                  dS_T=None, dd_T=None, scale=1.0, out=None, workspace=None):
    """Backward of osdn_forward on the GPU: the gradient of
    sum <dout, o> + <dS_T, S_T> + <dd_T, d_T> with respect to every input.

    Inputs as in osdn_forward; dout [B,H,T,Dv] in the dtype of q; dS_T
    [B,H,Dv,Dk] and dd_T [B,H,Dk] fp32 (None: zero). Returns a dict of fp32
    tensors q, k, v [B,H,T,*], beta, r [B,H,T], eta [B,H] (per stream; sum
    it for the shared scalar), d0 [B,H,Dk], S0 [B,H,Dv,Dk]. ``out`` may pass
    such a dict preallocated and ``workspace`` a uint8 device buffer of
    backward_workspace_bytes().
    """
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    f32 = torch.float32
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), f32, dev)
    _check(r, "r", (B, H, T), f32, dev)
    _check(d0, "d0", (B, H, Dk), f32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), f32, dev)
    _check(dout, "dout", (B, H, T, Dv), dt, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), f32, dev)
    _check(dd_T, "dd_T", (B, H, Dk), f32, dev)
    shapes = dict(q=(B, H, T, Dk), k=(B, H, T, Dk), v=(B, H, T, Dv),
                  beta=(B, H, T), r=(B, H, T), eta=(B, H), d0=(B, H, Dk),
                  S0=(B, H, Dv, Dk))
    g = out if out is not None else {
        n: torch.empty(s, dtype=f32, device=dev) for n, s in shapes.items()}
    for n, s in shapes.items():
        if g.get(n) is None:
            raise ValueError("out must hold a tensor for %s" % n)
        _check(g[n], "out[%s]" % n, s, f32, dev)
    need = L.osdn_backward_workspace_bytes(B, H, T, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.osdn_backward(B, H, T, Dk, Dv, _DTYPE_CODE[dt], _ptr(q), _ptr(k),
                         _ptr(v), _ptr(beta), _ptr(r), float(eta), _ptr(d0),
                         _ptr(S0), float(scale), _ptr(dout), _ptr(dS_T),
                         _ptr(dd_T), _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]),
                         _ptr(g["beta"]), _ptr(g["r"]), _ptr(g["eta"]),
                         _ptr(g["d0"]), _ptr(g["S0"]), _ptr(workspace),
                         workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_backward")
    return g


def _grad_outputs(out, shapes, dev):
    f32 = torch.float32
    g = out if out is not None else {
        n: torch.empty(s, dtype=f32, device=dev) for n, s in shapes.items()}
    for n, s in shapes.items():
        if g.get(n) is None:
            raise ValueError("out must hold a tensor for %s" % n)
        _check(g[n], "out[%s]" % n, s, f32, dev)
    return g


def gated_backward_workspace_bytes(B, H, T, Dk, Dv):
    return int(load_library().osdn_gated_backward_workspace_bytes(B, H, T, Dk,
                                                                  Dv))


def gdn2_backward_workspace_bytes(B, H, T, Dk, Dv):
    return int(load_library().gdn2_backward_workspace_bytes(B, H, T, Dk, Dv))


def osdn_gated_backward(q, k, v, beta, log_alpha, dout, r=None, eta=0.1,
                        d0=None, S0=None, dS_T=None, dd_T=None, scale=1.0,
                        out=None, workspace=None):
    """Backward of osdn_gated_forward on the GPU: as osdn_backward, with the
    per-channel decay log_alpha [B,H,T,Dk] fp32; the returned dict also holds
    log_alpha's gradient."""
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    f32 = torch.float32
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), f32, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), f32, dev)
    _check(r, "r", (B, H, T), f32, dev)
    _check(d0, "d0", (B, H, Dk), f32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), f32, dev)
    _check(dout, "dout", (B, H, T, Dv), dt, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), f32, dev)
    _check(dd_T, "dd_T", (B, H, Dk), f32, dev)
    g = _grad_outputs(out, dict(q=(B, H, T, Dk), k=(B, H, T, Dk),
                                v=(B, H, T, Dv), beta=(B, H, T), r=(B, H, T),
                                eta=(B, H), log_alpha=(B, H, T, Dk),
                                d0=(B, H, Dk), S0=(B, H, Dv, Dk)), dev)
    need = L.osdn_gated_backward_workspace_bytes(B, H, T, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.osdn_gated_backward(
        B, H, T, Dk, Dv, _DTYPE_CODE[dt], _ptr(q), _ptr(k), _ptr(v),
        _ptr(beta), _ptr(r), float(eta), _ptr(log_alpha), _ptr(d0), _ptr(S0),
        float(scale), _ptr(dout), _ptr(dS_T), _ptr(dd_T), _ptr(g["q"]),
        _ptr(g["k"]), _ptr(g["v"]), _ptr(g["beta"]), _ptr(g["r"]),
        _ptr(g["eta"]), _ptr(g["log_alpha"]), _ptr(g["d0"]), _ptr(g["S0"]),
        _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_gated_backward")
    return g


def gdn2_backward(q, k, v, log_alpha, b, w, dout, S0=None, dS_T=None,
                  scale=1.0, out=None, workspace=None):
    """Backward of gdn2_forward on the GPU: the gradient of
    sum <dout, o> + <dS_T, S_T>. Inputs as in gdn2_forward; dout [B,H,T,Dv]
    in the dtype of q, dS_T [B,H,Dk,Dv] fp32 (None: zero). Returns a dict of
    fp32 tensors q, k, log_alpha, b [B,H,T,Dk], v, w [B,H,T,Dv] and S0
    [B,H,Dk,Dv]."""
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a HIP device")
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    f32 = torch.float32
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), f32, dev)
    _check(b, "b", (B, H, T, Dk), dt, dev)
    _check(w, "w", (B, H, T, Dv), dt, dev)
    _check(S0, "S0", (B, H, Dk, Dv), f32, dev)
    _check(dout, "dout", (B, H, T, Dv), dt, dev)
    _check(dS_T, "dS_T", (B, H, Dk, Dv), f32, dev)
    g = _grad_outputs(out, dict(q=(B, H, T, Dk), k=(B, H, T, Dk),
                                v=(B, H, T, Dv), log_alpha=(B, H, T, Dk),
                                b=(B, H, T, Dk), w=(B, H, T, Dv),
                                S0=(B, H, Dk, Dv)), dev)
    need = L.gdn2_backward_workspace_bytes(B, H, T, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.gdn2_backward(
        B, H, T, Dk, Dv, _DTYPE_CODE[dt], _ptr(q), _ptr(k), _ptr(v),
        _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), float(scale),
        _ptr(dout), _ptr(dS_T), _ptr(g["q"]), _ptr(g["k"]), _ptr(g["v"]),
        _ptr(g["log_alpha"]), _ptr(g["b"]), _ptr(g["w"]), _ptr(g["S0"]),
        _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "gdn2_backward")
    return g


def precond_workspace_bytes(B, H, T, Dk, dtype):
    return int(load_library().osdn_precond_workspace_bytes(
        B, H, T, Dk, _DTYPE_CODE[dtype]))


def osdn_precond_scan(k, beta, r=None, eta=0.1, d0=None, want_ktilde=True,
                      out=None, workspace=None, diagnostics=False):
    """Phase 1 alone on the GPU: returns (ktilde or None, d_T), and with
    ``diagnostics=True`` also (rho, q_geo) as in osdn_forward.

    ``out`` may pass preallocated (ktilde, d_T) (ktilde may be None to skip
    it) and ``workspace`` a preallocated uint8 device buffer.
    """
    L = load_library()
    dev = k.device
    B, H, T, Dk = k.shape
    dt = k.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(r, "r", (B, H, T), torch.float32, dev)
    _check(d0, "d0", (B, H, Dk), torch.float32, dev)
    if out is None:
        kt = torch.empty_like(k) if want_ktilde else None
        d_T = torch.empty((B, H, Dk), dtype=torch.float32, device=dev)
    else:
        kt, d_T = out
    _check(kt, "ktilde", (B, H, T, Dk), dt, dev)
    _check(d_T, "d_T", (B, H, Dk), torch.float32, dev)
    need = L.osdn_precond_workspace_bytes(B, H, T, Dk, _DTYPE_CODE[dt])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rho = qg = None
    if diagnostics:
        rho = torch.empty((B, H, T), dtype=torch.float32, device=dev)
        qg = torch.empty((B, H), dtype=torch.float32, device=dev)
    rc = L.osdn_precond_scan(B, H, T, Dk, _DTYPE_CODE[dt], _ptr(k), _ptr(beta),
                             _ptr(r), float(eta), _ptr(d0), _ptr(kt), _ptr(d_T),
                             _ptr(rho), _ptr(qg), _ptr(workspace),
                             workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_precond_scan")
    if diagnostics:
        return kt, d_T, rho, qg
    return kt, d_T


def osdn_chunk_forward(q, k, ktilde, v, beta, S0=None, chunk=64, scale=1.0,
                       out=None, workspace=None):
    """Phase 2 alone on the GPU (write keys ktilde given): returns (o, S_T)."""
    L = load_library()
    dev = q.device
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (ktilde, "ktilde")):
        _check(t, n, (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if out is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    else:
        o, S_T = out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    _check(S_T, "S_T", (B, H, Dv, Dk), torch.float32, dev)
    need = L.osdn_chunk_workspace_bytes(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.osdn_chunk_forward(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt], _ptr(q),
                              _ptr(k), _ptr(ktilde), _ptr(v), _ptr(beta),
                              _ptr(S0), float(scale), _ptr(o), _ptr(S_T),
                              _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_chunk_forward")
    return o, S_T


def gdn2_forward(q, k, v, log_alpha, b, w, S0=None, chunk=64, scale=1.0,
                 out=None, workspace=None):
    """Gated DeltaNet-2 forward on the GPU: returns (o, S_T).

    q, k, b: [B,H,T,Dk]; v, w: [B,H,T,Dv] (one dtype, fp32 or bf16);
    log_alpha: [B,H,T,Dk] fp32; S0: [B,H,Dk,Dv] fp32 (None: zeros).
    """
    L = load_library()
    dev = q.device
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    for t, n in ((q, "q"), (k, "k"), (b, "b")):
        _check(t, n, (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(w, "w", (B, H, T, Dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), torch.float32, dev)
    _check(S0, "S0", (B, H, Dk, Dv), torch.float32, dev)
    if out is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    else:
        o, S_T = out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    _check(S_T, "S_T", (B, H, Dk, Dv), torch.float32, dev)
    need = L.gdn2_forward_workspace_bytes(B, H, T, Dk, Dv, chunk,
                                          _DTYPE_CODE[dt])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.gdn2_forward(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt], _ptr(q),
                        _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                        _ptr(S0), float(scale), _ptr(o), _ptr(S_T),
                        _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "gdn2_forward")
    return o, S_T


def osdn_decode(q, k, v, beta, S, d, r=None, eta=0.1, scale=1.0, out=None,
                log_alpha=None):
    """OSDN recurrent decode on the GPU: advances the T tokens of q, k, v
    (usually T = 1) through the token recurrence, updating S ([B,H,Dv,Dk]
    fp32) and d ([B,H,Dk] fp32) IN PLACE; returns o [B,H,T,Dv].
    log_alpha ([B,H,T,Dk] fp32): per-channel decay of a gated backbone, as
    in osdn_gated_forward (None: plain OSDN)."""
    L = load_library()
    dev = q.device
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(r, "r", (B, H, T), torch.float32, dev)
    _check(S, "S", (B, H, Dv, Dk), torch.float32, dev)
    _check(d, "d", (B, H, Dk), torch.float32, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), torch.float32, dev)
    o = torch.empty((B, H, T, Dv), dtype=dt, device=dev) if out is None else out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    rc = L.osdn_decode(B, H, T, Dk, Dv, _DTYPE_CODE[dt], _ptr(q), _ptr(k),
                       _ptr(v), _ptr(beta), _ptr(r), float(eta),
                       _ptr(log_alpha), _ptr(S), _ptr(d), float(scale),
                       _ptr(o), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_decode")
    return o


def gdn2_decode(q, k, v, log_alpha, b, w, S, scale=1.0, out=None):
    """Gated DeltaNet-2 recurrent decode on the GPU: T tokens with the state
    S ([B,H,Dk,Dv] fp32) updated IN PLACE; returns o [B,H,T,Dv]."""
    L = load_library()
    dev = q.device
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    for t, n in ((q, "q"), (k, "k"), (b, "b")):
        _check(t, n, (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(w, "w", (B, H, T, Dv), dt, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), torch.float32, dev)
    _check(S, "S", (B, H, Dk, Dv), torch.float32, dev)
    o = torch.empty((B, H, T, Dv), dtype=dt, device=dev) if out is None else out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    rc = L.gdn2_decode(B, H, T, Dk, Dv, _DTYPE_CODE[dt], _ptr(q), _ptr(k),
                       _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S),
                       float(scale), _ptr(o), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "gdn2_decode")
    return o


def osdn_gated_forward(q, k, v, beta, log_alpha, r=None, eta=0.1, d0=None,
                       S0=None, chunk=64, scale=1.0, out=None, workspace=None):
    """OSDN on a per-key-channel-decay backbone on the GPU: returns
    (o, S_T, d_T). Arguments as for osdn_forward plus log_alpha
    [B,H,T,Dk] fp32 (the decay applied to the state before each token's
    step)."""
    L = load_library()
    if q.dtype not in _DTYPE_CODE:
        raise ValueError("q, k, v must be float32 or bfloat16")
    dev = q.device
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dt = q.dtype
    _check(q, "q", (B, H, T, Dk), dt, dev)
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(beta, "beta", (B, H, T), torch.float32, dev)
    _check(r, "r", (B, H, T), torch.float32, dev)
    _check(log_alpha, "log_alpha", (B, H, T, Dk), torch.float32, dev)
    _check(d0, "d0", (B, H, Dk), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    if out is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
        d_T = torch.empty((B, H, Dk), dtype=torch.float32, device=dev)
    else:
        o, S_T, d_T = out
    _check(o, "o", (B, H, T, Dv), dt, dev)
    _check(S_T, "S_T", (B, H, Dv, Dk), torch.float32, dev)
    _check(d_T, "d_T", (B, H, Dk), torch.float32, dev)
    need = L.osdn_gated_forward_workspace_bytes(B, H, T, Dk, Dv, chunk,
                                                _DTYPE_CODE[dt])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = L.osdn_gated_forward(B, H, T, Dk, Dv, chunk, _DTYPE_CODE[dt],
                              _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(r),
                              float(eta), _ptr(log_alpha), _ptr(d0), _ptr(S0),
                              float(scale), _ptr(o), _ptr(S_T), _ptr(d_T),
                              _ptr(workspace), workspace.numel(), _stream(dev))
    if rc != 0:
        raise OsdnError(rc, "osdn_gated_forward")
    return o, S_T, d_T
