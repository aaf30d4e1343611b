"""bench.py's measurement contract on the CPU: the one-GPU refusal, and the
algorithmic bytes and flops its roofline divides by, each written out here
tensor by tensor at the 1.3B-layer shape (B=4, H=16, T=4096, Dk=Dv=128,
bf16, forgetting gate on)."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_forward_path_bytes_at_the_headline_shape():
    w = W.BY_NAME["osdn-1.3b-apf"]
    assert (w.B, w.H, w.T, w.Dk, w.Dv, w.dtype, w.apf) == (4, 16, 4096, 128, 128,
                                                            "bf16", True)
    token_heads, streams = 4 * 16 * 4096, 4 * 16
    per_token = (128 * 2      # q, bf16
                 + 128 * 2    # k
                 + 128 * 2    # v
                 + 128 * 2    # o written
                 + 4          # beta, fp32
                 + 4)         # r, fp32
    per_stream = (128 * 128 * 4   # S_T written, fp32
                  + 128 * 4       # d0 read
                  + 128 * 4)      # d_T written
    assert per_token == 1032
    assert bench.path_bytes(w) == token_heads * per_token + streams * per_stream
    assert bench.path_bytes(w) == 274_792_448


def test_gdn2_and_gated_path_bytes():
    g = W.BY_NAME["gdn2-1.3b"]
    per_token = (3 * 128 * 2      # q, k, b (bf16)
                 + 2 * 128 * 2    # v, w
                 + 128 * 4        # log alpha, fp32
                 + 128 * 2)       # o
    assert bench.path_bytes(g) == 4 * 16 * 4096 * per_token + 64 * 128 * 128 * 4
    o = W.BY_NAME["osdn-gated-1.3b"]
    assert bench.path_bytes(o) == (bench.path_bytes(W.BY_NAME["osdn-1.3b-apf"])
                                   + 4 * 16 * 4096 * 128 * 4)   # + log alpha


def test_decode_bytes_per_head():
    w = W.BY_NAME["osdn-decode"]
    assert w.T == 1 and w.Dk == w.Dv == 128 and w.apf
    state = 2 * 128 * 128 * 4                   # S read and written
    precond = 2 * 128 * 4                       # d read and written
    token = 4 * 128 * 2 + 4 + 4                 # q, k, v, o; beta, r
    assert bench.decode_bytes_per_head(w) == state + precond + token


def test_chunk_form_flops_per_token_head():
    w = W.BY_NAME["osdn-1.3b-apf"]
    C, d = 64, 128
    state_chain = 4 * d * d           # W = U - Wk S^T and S += W^T X'
    inter_chunk = 2 * d * d           # Q S^T
    intra = 2 * C * (3 * d + 2 * d)   # Gram, Wk, scores; U, P W
    inverse = C * C / 3.0
    assert abs(bench.flops_per_token_head(w)
               - (state_chain + inter_chunk + intra + inverse)) < 1e-9
    assert round(bench.flops_per_token_head(w)) == 181_589


def test_backward_bytes_at_the_headline_shape():
    w = W.BY_NAME["osdn-1.3b-apf"]
    per_token = (3 * 128 * 2 + 4 + 4   # q, k, v; beta, r read
                 + 128 * 2             # do read
                 + (3 * 128 + 2) * 4)  # dq, dk, dv, dbeta, dr written (fp32)
    per_stream = (128 * 128 * 4 * 2    # dS_T read, dS0 written
                  + 128 * 4 * 2        # dd_T read, dd0 written
                  + 4)                 # deta written
    assert bench.backward_bytes(w) == 4 * 16 * 4096 * per_token + 64 * per_stream
