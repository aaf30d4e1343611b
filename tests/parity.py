"""Error measures shared by the GPU parity tests (not a test module).

The pages' bound is a relative L2 error over the compared tensor,
||x - ref|| / ||ref||: 1e-4 on the fp32 path, 2e-2 on the bf16-input /
fp32-state path, 1e-5 for the preconditioner d. The chunked GPU form is an
exact rewrite of the token recurrence, so its differences are rounding only;
rounding is spread evenly over streams and tokens, which the finer measures
below hold it to:

* per stream: the relative L2 error of every (batch, head) stream on its own
  must meet the tensor bound (a wrong stream cannot hide among correct ones);
* per token: the error of each output row t of a stream, relative to that
  row's norm plus the stream's RMS row norm (rows near zero do not blow it
  up), must stay within TOKEN_FACTOR times the tensor bound, and the largest
  element error within MAXABS_FACTOR times the tensor bound of the stream's
  largest reference element (one wrong row among T = 4096 moves the tensor
  figure by only about 1/T of its own error).
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}
D_TOL = 1e-5
TOKEN_FACTOR = 5.0
MAXABS_FACTOR = 5.0


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def per_stream_rel_l2(x, ref):
    """[B, H] relative L2 error of each (batch, head) stream."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    B, H = ref.shape[:2]
    d = (x - ref).reshape(B, H, -1)
    r = ref.reshape(B, H, -1)
    num = np.linalg.norm(d, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    return num / np.where(den > 0, den, 1.0)


def per_token(x, ref):
    """(row error [B, H, T], element error [B, H]) of an output [B, H, T, D]:
    row error ||x_t - ref_t|| / (||ref_t|| + rms_t ||ref_t||); element error
    max |x - ref| / max |ref| per stream."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rn = np.linalg.norm(ref, axis=-1)
    rms = np.sqrt(np.mean(rn * rn, axis=-1, keepdims=True))
    row = np.linalg.norm(x - ref, axis=-1) / np.maximum(rn + rms, 1e-300)
    B, H = ref.shape[:2]
    amax = np.abs(ref).reshape(B, H, -1).max(axis=-1)
    emax = np.abs(x - ref).reshape(B, H, -1).max(axis=-1)
    return row, emax / np.where(amax > 0, amax, 1.0)


def check_full(where, dtype, o, ro, S, rS, d=None, rd=None):
    """Whole-tensor, per-stream and per-token checks of (o, S_T[, d_T])."""
    tol = TOL[dtype]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    eo, eS = rel_l2(o, ro), rel_l2(S, rS)
    so, sS = per_stream_rel_l2(o, ro), per_stream_rel_l2(S, rS)
    row, elem = per_token(o, ro) if o.shape[2] > 0 else (np.zeros(1), np.zeros(1))
    msg = ("%s: rel_l2 o=%.3e S_T=%.3e | worst stream o=%.3e S_T=%.3e | "
           "worst token row %.3e, worst element %.3e"
           % (where, eo, eS, so.max(), sS.max(), row.max(), elem.max()))
    if d is not None:
        ed = rel_l2(d, rd)
        sd = per_stream_rel_l2(d, rd)
        msg += " | d_T=%.3e worst stream %.3e" % (ed, sd.max())
    print(msg, flush=True)
    assert eo <= tol and eS <= tol, msg
    assert so.max() <= tol and sS.max() <= tol, msg
    assert row.max() <= TOKEN_FACTOR * tol, msg
    assert elem.max() <= MAXABS_FACTOR * tol, msg
    if d is not None:
        assert np.all(np.isfinite(d))
        assert ed <= D_TOL and sd.max() <= D_TOL, msg
