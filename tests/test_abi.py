"""C-ABI checks that need no GPU: the library loads, exports every symbol the
headers declare, and rejects bad arguments on the host before any launch.

Every call here fails host-side validation, so no HIP work is enqueued.
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import delta_rule_recurrent_scan_amd as osdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = osdn.library_path()

OK, NULL_ARG, BAD_DIMS, UNSUPPORTED, WORKSPACE, ALIASING, HIP = range(7)

needs_lib = pytest.mark.skipif(not os.path.exists(LIB),
                               reason="libosdn.so not built")


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*"
                            r"([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("osdn_forward", "osdn_forward_workspace_bytes", "osdn_strerror",
              "osdn_forward_supported", "osdn_precond_scan",
              "osdn_precond_workspace_bytes",
              "osdn_chunk_forward", "gdn2_forward", "gdn2_forward_supported",
              "osdn_chunk_workspace_bytes", "gdn2_forward_workspace_bytes",
              "osdn_decode", "gdn2_decode", "osdn_gated_forward",
              "osdn_gated_forward_workspace_bytes",
              "osdn_gated_forward_supported"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (\S+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, "declared but not exported: %s" % missing
    L = osdn.load_library()
    for n in declared_functions():
        assert hasattr(L, n)


@needs_lib
def test_strerror():
    L = osdn.load_library()
    for s in range(7):
        assert L.osdn_strerror(s)
    assert L.osdn_strerror(99) == b"unknown status"


@needs_lib
def test_supported_and_workspace_sizes():
    L = osdn.load_library()
    for dk in (32, 64, 128):
        for dv in (32, 64, 128):
            for c in (16, 32, 64):
                assert L.osdn_forward_supported(dk, dv, c, 1) == 1
    assert L.osdn_forward_supported(32, 32, 16, 0) == 1
    assert L.osdn_forward_supported(48, 32, 16, 1) == 0
    assert L.osdn_forward_supported(32, 32, 8, 1) == 0
    assert L.osdn_forward_supported(32, 32, 16, 7) == 0
    # phase-1 scratch: per 64-token chunk, lp (64 + 4), g (64), V (64 x 64),
    # the gate ratios (64 + 4) and the entry value of d (Dk), all fp32;
    # rounded up to 256 bytes
    def pre(BH, T, Dk):
        n = BH * ((T + 63) // 64) * (68 + 64 + 64 * 64 + 68 + Dk) * 4
        return (n + 255) // 256 * 256
    assert L.osdn_precond_workspace_bytes(4, 16, 4096, 128, 1) == pre(64, 4096, 128)
    assert L.osdn_precond_workspace_bytes(1, 1, 0, 32, 1) == 0
    assert L.osdn_precond_workspace_bytes(1, 1, 8, 40, 1) == 0
    # chunk engine: per chunk, Wk, X' (Dk columns), U (Dv columns) and the
    # scores P (C columns) in the storage dtype; GDN-2 adds its decayed
    # queries (Dk columns) and the exit decay (Dk fp32)
    def wy(BH, T, Dk, Dv, C, es, gdn2=False):
        nc = BH * ((T + C - 1) // C)
        n = nc * C * ((3 if gdn2 else 2) * Dk + Dv + C) * es
        if gdn2:
            n += nc * Dk * 4
        return (n + 255) // 256 * 256
    assert L.osdn_chunk_workspace_bytes(4, 16, 4096, 128, 128, 64, 1) == \
        wy(64, 4096, 128, 128, 64, 2)
    assert L.gdn2_forward_workspace_bytes(2, 3, 100, 64, 32, 32, 0) == \
        wy(6, 100, 64, 32, 32, 4, gdn2=True)
    # chunk 64: both scratch regions (phase 2 forms K~ from the records);
    # other chunks: K~ plus the larger of the two
    assert L.osdn_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, 1) == \
        pre(64, 4096, 128) + wy(64, 4096, 128, 128, 64, 2)
    assert L.osdn_forward_workspace_bytes(1, 1, 3, 32, 32, 16, 0) == \
        512 + max(pre(1, 3, 32), wy(1, 3, 32, 32, 16, 4))
    assert L.osdn_forward_workspace_bytes(-1, 1, 3, 32, 32, 16, 0) == 0


def _fwd(L, B=1, H=1, T=64, Dk=32, Dv=32, C=16, dt=1, q=0x10000, k=0x20000,
         v=0x30000, beta=0x40000, r=None, d0=None, S0=None, o=0x50000,
         ST=None, dT=None, rho=None, qg=None, ws=0x100000, wsb=1 << 20):
    P = ctypes.c_void_p
    L.osdn_forward.argtypes = ([ctypes.c_int] * 7 +
                               [P, P, P, P, P, ctypes.c_float, P, P,
                                ctypes.c_float, P, P, P, P, P, P,
                                ctypes.c_size_t, P])
    return L.osdn_forward(B, H, T, Dk, Dv, C, dt, q, k, v, beta, r, 0.1, d0,
                          S0, 1.0, o, ST, dT, rho, qg, ws, wsb, None)


@needs_lib
def test_error_paths_are_host_side():
    L = osdn.load_library()
    assert _fwd(L, q=None) == NULL_ARG
    assert _fwd(L, beta=None) == NULL_ARG
    assert _fwd(L, o=None) == NULL_ARG
    assert _fwd(L, T=-1) == BAD_DIMS
    assert _fwd(L, B=-2) == BAD_DIMS
    assert _fwd(L, Dk=48) == UNSUPPORTED
    assert _fwd(L, C=8) == UNSUPPORTED
    assert _fwd(L, dt=5) == UNSUPPORTED
    assert _fwd(L, ws=None) == WORKSPACE
    assert _fwd(L, wsb=100) == WORKSPACE
    assert _fwd(L, ws=0x100010) == WORKSPACE          # not 256-byte aligned
    # o overlapping v; S_T overlapping q; workspace overlapping k
    assert _fwd(L, o=0x30000 + 64) == ALIASING
    assert _fwd(L, ST=0x10000 + 8) == ALIASING
    assert _fwd(L, ws=0x20000) == ALIASING
    # partial overlap of S_T with S0 is rejected (exact aliasing would pass)
    assert _fwd(L, S0=0x200000, ST=0x200000 + 4) == ALIASING
    assert _fwd(L, d0=0x300000, dT=0x300000 + 4) == ALIASING
    # the residual-ratio outputs are outputs like the others
    assert _fwd(L, rho=0x40000 + 8) == ALIASING      # over beta
    assert _fwd(L, qg=0x50000) == ALIASING           # over o
    assert _fwd(L, rho=0x400000, qg=0x400000 + 16) == ALIASING


@needs_lib
def test_precond_scan_error_paths():
    L = osdn.load_library()
    P = ctypes.c_void_p
    L.osdn_precond_scan.argtypes = [ctypes.c_int] * 5 + [P, P, P, ctypes.c_float,
                                                         P, P, P, P, P, P,
                                                         ctypes.c_size_t, P]

    def pre(B=1, T=8, Dk=32, k=0x1000, beta=0x2000, kt=None, dT=None,
            rho=None, qg=None, ws=0x100000, wsb=1 << 20):
        return L.osdn_precond_scan(B, 1, T, Dk, 1, k, beta, None, 0.1, None,
                                   kt, dT, rho, qg, ws, wsb, None)
    assert pre(k=None) == NULL_ARG
    assert pre(T=-8) == BAD_DIMS
    assert pre(Dk=40) == UNSUPPORTED
    assert pre(ws=None) == WORKSPACE
    assert pre(wsb=64) == WORKSPACE
    assert pre(ws=0x100040) == WORKSPACE          # not 256-byte aligned
    assert pre(kt=0x1000 + 16) == ALIASING
    assert pre(ws=0x1000) == ALIASING             # workspace over k
    assert pre(rho=0x2000) == ALIASING            # rho over beta
    assert pre(qg=0x100000 + 256) == ALIASING     # q_geo inside the workspace
    # B = 0: nothing to do, no pointer or workspace needed
    assert pre(B=0, k=None, beta=None, ws=None, wsb=0) == OK


@needs_lib
def test_kernel_timing_host_side():
    # with nothing launched the record is empty (no HIP call is made)
    osdn.kernel_timing(True)
    assert osdn.kernel_times() == {}
    osdn.kernel_timing(False)
    assert osdn.load_library().osdn_kernel_times(0, None, None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(osdn, "_lib", None)
    monkeypatch.setattr(osdn, "_LIB_PATH", "/nonexistent/libosdn.so")
    with pytest.raises(RuntimeError, match="not built"):
        osdn.load_library()


@needs_lib
def test_gdn2_error_paths():
    L = osdn.load_library()
    P = ctypes.c_void_p
    L.gdn2_forward.argtypes = [ctypes.c_int] * 7 + [P] * 7 + [ctypes.c_float,
                                                              P, P, P,
                                                              ctypes.c_size_t, P]

    def call(T=64, Dk=32, q=0x10000, la=0x60000, o=0x50000, ST=None, S0=None,
             ws=0x100000, wsb=1 << 20):
        return L.gdn2_forward(1, 1, T, Dk, 32, 16, 1, q, 0x20000, 0x30000, la,
                              0x70000, 0x80000, S0, 1.0, o, ST, ws, wsb, None)

    assert call(q=None) == NULL_ARG
    assert call(la=None) == NULL_ARG
    assert call(T=-3) == BAD_DIMS
    assert call(Dk=48) == UNSUPPORTED
    assert call(o=0x20000 + 128) == ALIASING
    assert call(S0=0x200000, ST=0x200000 + 8) == ALIASING
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(ws=0x30000) == ALIASING          # workspace over v
    assert L.gdn2_forward_supported(128, 128, 64, 1) == 1
    assert L.gdn2_forward_supported(128, 128, 8, 1) == 0


@needs_lib
def test_decode_error_paths():
    L = osdn.load_library()
    P = ctypes.c_void_p
    I, F = ctypes.c_int, ctypes.c_float
    L.osdn_decode.argtypes = [I] * 6 + [P, P, P, P, P, F, P, P, P, F, P, P]
    L.gdn2_decode.argtypes = [I] * 6 + [P] * 7 + [F, P, P]

    def dec(B=2, T=1, Dk=32, q=0x10000, beta=0x40000, S=0x200000, d=0x300000,
            o=0x50000, r=None, la=None):
        return L.osdn_decode(B, 1, T, Dk, 32, 1, q, 0x20000, 0x30000, beta, r,
                             0.1, la, S, d, 1.0, o, None)
    assert dec(q=None) == NULL_ARG
    assert dec(S=None) == NULL_ARG
    assert dec(d=None) == NULL_ARG
    assert dec(T=-1) == BAD_DIMS
    assert dec(Dk=48) == UNSUPPORTED
    assert dec(S=0x10000 + 4) == ALIASING        # state over q
    assert dec(d=0x200000 + 64) == ALIASING      # d inside the state
    assert dec(o=0x300000) == ALIASING           # o over d
    assert dec(r=0x200000) == ALIASING           # gate over the state
    assert dec(la=0x300000 + 16) == ALIASING     # decay over d
    # nothing to do: T = 0 or B = 0 needs no pointer
    assert dec(T=0, q=None, S=None, d=None, o=None, beta=None) == OK
    assert dec(B=0, q=None, S=None, d=None, o=None, beta=None) == OK

    def gd(T=1, Dv=32, la=0x60000, S=0x200000, o=0x50000):
        return L.gdn2_decode(1, 1, T, 32, Dv, 1, 0x10000, 0x20000, 0x30000,
                             la, 0x70000, 0x80000, S, 1.0, o, None)
    assert gd(la=None) == NULL_ARG
    assert gd(S=None) == NULL_ARG
    assert gd(T=-2) == BAD_DIMS
    assert gd(Dv=16) == UNSUPPORTED
    assert gd(S=0x70000) == ALIASING             # state over b
    assert gd(o=0x200000 + 8) == ALIASING        # o inside the state
    assert gd(T=0, la=None, S=None, o=None) == OK


@needs_lib
def test_gated_forward_error_paths_and_workspace():
    L = osdn.load_library()
    P = ctypes.c_void_p
    I, F = ctypes.c_int, ctypes.c_float
    L.osdn_gated_forward.argtypes = ([I] * 7 + [P, P, P, P, P, F, P, P, P, F, P,
                                                P, P, P, ctypes.c_size_t, P])

    def call(T=64, Dk=32, C=16, la=0x60000, o=0x50000, ST=None, S0=None,
             ws=0x100000, wsb=1 << 20):
        return L.osdn_gated_forward(1, 1, T, Dk, 32, C, 1, 0x10000, 0x20000,
                                    0x30000, 0x40000, None, 0.1, la, None, S0,
                                    1.0, o, ST, None, ws, wsb, None)
    assert call(la=None) == NULL_ARG
    assert call(T=-1) == BAD_DIMS
    assert call(Dk=48) == UNSUPPORTED
    assert call(Dk=32, C=8) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(o=0x60000 + 64) == ALIASING      # o over log alpha
    assert call(S0=0x200000, ST=0x200000 + 4) == ALIASING
    assert call(ws=0x30000) == ALIASING          # workspace over v
    # chunk 64 (bf16): both scratch regions, the engine forms K~ itself;
    # other chunks: the preconditioned keys, then the larger of the two
    def r256(n):
        return (n + 255) // 256 * 256
    kt = r256(64 * 4096 * 128 * 2)
    p1 = L.osdn_precond_workspace_bytes(4, 16, 4096, 128, 1)
    p2 = L.gdn2_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, 1)
    assert L.osdn_gated_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, 1) \
        == p1 + p2
    p2b = L.gdn2_forward_workspace_bytes(4, 16, 4096, 128, 128, 32, 1)
    assert L.osdn_gated_forward_workspace_bytes(4, 16, 4096, 128, 128, 32, 1) \
        == kt + max(p1, p2b)
    assert L.osdn_gated_forward_supported(128, 128, 64, 1) == 1
    assert L.osdn_gated_forward_supported(128, 128, 8, 1) == 0


def _layout_bytes(L, B, H, T, Dk, Dv, C, dt, gated):
    """Bytes a two-phase forward touches, by the layout rule the header
    states: fused (chunk 64; for the gated forward where its fused engine
    layout fits) = phase-1 scratch + phase-2 scratch; otherwise K~ (rounded
    up to 256 bytes) + the larger of the two."""
    r256 = lambda n: (n + 255) // 256 * 256
    p1 = L.osdn_precond_workspace_bytes(B, H, T, Dk, dt)
    if gated:
        p2 = L.gdn2_forward_workspace_bytes(B, H, T, Dk, Dv, C, dt)
        fused = C == 64 and (dt == 1 or Dk == 32 or (Dk == 64 and Dv <= 64))
    else:
        p2 = L.osdn_chunk_workspace_bytes(B, H, T, Dk, Dv, C, dt)
        fused = C == 64
    if fused:
        return p1 + p2
    return r256(B * H * T * Dk * (2 if dt == 1 else 4)) + max(p1, p2)


@needs_lib
@pytest.mark.parametrize("gated", [False, True])
def test_workspace_covers_every_supported_size(gated):
    """For every (Dk, Dv, chunk, dtype) with a kernel instance and several
    (B, H, T), the advertised workspace equals the bytes the call's layout
    places (so it covers every region it touches); unsupported sizes
    advertise 0. This includes fp32 at chunk 64, whose query once chose the
    gated engine's layout rule and came out short."""
    L = osdn.load_library()
    sup = L.osdn_gated_forward_supported if gated else L.osdn_forward_supported
    query = (L.osdn_gated_forward_workspace_bytes if gated
             else L.osdn_forward_workspace_bytes)
    seen = 0
    for dt in (0, 1):
        for dk in (32, 64, 128):
            for dv in (32, 64, 128):
                for c in (16, 32, 64):
                    for B, H, T in ((1, 1, 1), (2, 3, 448), (4, 16, 4096),
                                    (1, 2, 63), (3, 1, 1000)):
                        got = query(B, H, T, dk, dv, c, dt)
                        if not sup(dk, dv, c, dt):
                            assert got == 0, (dt, dk, dv, c)
                            continue
                        need = _layout_bytes(L, B, H, T, dk, dv, c, dt, gated)
                        assert got == need, (dt, dk, dv, c, B, H, T, got, need)
                        assert got % 256 == 0
                        seen += 1
    assert seen > 100


@needs_lib
def test_fp32_chunk64_workspace_regression():
    """fp32, Dk = Dv = 64, chunk 64, B=2 H=3 T=448: the call keeps the
    phase-1 records and the phase-2 operands side by side, which is more
    than the preconditioned keys plus the larger region (the short size the
    query once returned)."""
    L = osdn.load_library()
    assert L.osdn_forward_supported(64, 64, 64, 0) == 1
    p1 = L.osdn_precond_workspace_bytes(2, 3, 448, 64, 0)
    p2 = L.osdn_chunk_workspace_bytes(2, 3, 448, 64, 64, 64, 0)
    short = (2 * 3 * 448 * 64 * 4 + 255) // 256 * 256 + max(p1, p2)
    assert p1 + p2 > short
    assert L.osdn_forward_workspace_bytes(2, 3, 448, 64, 64, 64, 0) == p1 + p2


@needs_lib
def test_noalloc_rejects_sizes_beyond_its_scratch():
    """osdn_forward_noalloc checks the size against its static scratch before
    touching any device (the fake pointers below are never dereferenced)."""
    L = osdn.load_library()
    P = ctypes.c_void_p
    I, F = ctypes.c_int, ctypes.c_float
    L.osdn_forward_noalloc.argtypes = ([I] * 7 + [P, P, P, P, P, F, P, P, F,
                                                  P, P, P, P, P, P])
    cap = osdn.NOALLOC_SCRATCH_BYTES
    assert cap == 128 << 20
    # the 1.3B-layer workload needs about 300 MB of scratch: rejected
    assert L.osdn_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, 1) > cap
    args = (0x10000, 0x20000, 0x30000, 0x40000, None, 0.1, None, None, 1.0,
            0x50000, None, None, None, None, None)
    assert L.osdn_forward_noalloc(4, 16, 4096, 128, 128, 64, 1, *args) == WORKSPACE
    assert L.osdn_forward_noalloc(1, 1, 64, 48, 32, 16, 1, *args) == UNSUPPORTED
    assert L.osdn_forward_noalloc(1, 1, -1, 32, 32, 16, 1, *args) == BAD_DIMS
    # nothing to do: no pointer needed, no device touched
    assert L.osdn_forward_noalloc(0, 1, 64, 32, 32, 16, 1, *((None,) * 4),
                                  None, 0.1, None, None, 1.0, *((None,) * 5),
                                  None) == OK


@needs_lib
def test_backward_error_paths_and_workspace():
    L = osdn.load_library()
    P = ctypes.c_void_p
    I, F, Z = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.osdn_backward.argtypes = ([I] * 6 + [P, P, P, P, P, F, P, P, F, P, P, P]
                                + [P] * 8 + [P, Z, P])
    L.osdn_backward_workspace_bytes.argtypes = [I] * 5
    L.osdn_backward_workspace_bytes.restype = Z
    # per token u (Dv) and d (Dk), a state every 64 tokens and after the
    # last, and per token and 32-row value slice the slice's row sums
    # (3 Dk + 1, padded to 3 Dk + 4)
    for B, H, T, Dk, Dv in ((1, 1, 1, 32, 32), (2, 3, 64, 64, 128),
                            (1, 2, 65, 128, 32), (2, 1, 0, 32, 64)):
        nck = (T + 63) // 64
        want = B * H * (T * (Dk + Dv) + (nck + 1) * Dv * Dk
                        + T * (Dv // 32) * (3 * Dk + 4)) * 4
        assert L.osdn_backward_workspace_bytes(B, H, T, Dk, Dv) == want
    assert L.osdn_backward_workspace_bytes(1, 1, 8, 48, 32) == 0
    assert L.osdn_backward_workspace_bytes(-1, 1, 8, 32, 32) == 0

    ws_at = 0x4000000
    need = L.osdn_backward_workspace_bytes(1, 1, 4, 32, 32)

    def bwd(B=1, T=4, Dk=32, q=0x10000, dout=0x60000, dq=0x100000,
            dS0=0x900000, ws=ws_at, wsb=need, beta=0x40000, dST=None):
        return L.osdn_backward(B, 1, T, Dk, 32, 1, q, 0x20000, 0x30000, beta,
                               None, 0.1, None, None, 1.0, dout, dST, None,
                               dq, 0x200000, 0x300000, 0x400000, 0x500000,
                               0x600000, 0x700000, dS0, ws, wsb, None)
    assert bwd(q=None) == NULL_ARG
    assert bwd(dout=None) == NULL_ARG
    assert bwd(dS0=None) == NULL_ARG
    assert bwd(T=-1) == BAD_DIMS
    assert bwd(Dk=48) == UNSUPPORTED
    assert bwd(ws=None) == WORKSPACE
    assert bwd(wsb=need - 4) == WORKSPACE
    assert bwd(ws=ws_at + 16) == WORKSPACE       # not 256-byte aligned
    assert bwd(dq=0x10000 + 4) == ALIASING       # dq over q
    assert bwd(dq=0x200000 + 64) == ALIASING     # dq over dk
    assert bwd(dST=0x900000) == ALIASING         # dS0 over dS_T
    assert bwd(dS0=ws_at + 256) == ALIASING      # dS0 inside the workspace
    # no streams: nothing to do, no pointer needed
    assert bwd(B=0, q=None, dout=None, dq=None, dS0=None, ws=None,
               beta=None) == OK


@needs_lib
@pytest.mark.parametrize("gdn2", [False, True])
def test_gated_backward_error_paths_and_workspace(gdn2):
    L = osdn.load_library()
    P = ctypes.c_void_p
    I, F, Z = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.osdn_gated_backward.argtypes = ([I] * 6 + [P, P, P, P, P, F, P, P, P, F,
                                                 P, P, P] + [P] * 9 + [P, Z, P])
    L.gdn2_backward.argtypes = [I] * 6 + [P] * 7 + [F, P, P] + [P] * 7 + [P, Z, P]
    wsq = (L.gdn2_backward_workspace_bytes if gdn2
           else L.osdn_gated_backward_workspace_bytes)
    wsq.argtypes = [I] * 5
    wsq.restype = Z
    # OSDN: per token d (Dk); both: a state every 64 tokens and after the
    # last, an interval of min(T, 64) states, and per token and 32-row value
    # slice the slice's row sums (4 Dk + 4)
    for B, H, T, Dk, Dv in ((1, 1, 1, 32, 32), (2, 3, 64, 64, 128),
                            (1, 2, 130, 128, 32), (2, 1, 0, 32, 64)):
        nck = (T + 63) // 64
        per = ((0 if gdn2 else T * Dk) + (nck + 1 + min(T, 64)) * Dv * Dk
               + T * (Dv // 32) * (4 * Dk + 4))
        assert wsq(B, H, T, Dk, Dv) == B * H * per * 4
    assert wsq(1, 1, 8, 48, 32) == 0
    need = wsq(1, 1, 4, 32, 32)
    ws_at = 0x4000000

    def call(B=1, T=4, Dk=32, q=0x10000, la=0x80000, dq=0x100000,
             dS0=0x900000, ws=ws_at, wsb=need, dla=0xa00000):
        if gdn2:
            return L.gdn2_backward(B, 1, T, Dk, 32, 1, q, 0x20000, 0x30000, la,
                                   0x90000, 0x98000, None, 1.0, 0x60000, None,
                                   dq, 0x200000, 0x300000, dla, 0x400000,
                                   0x500000, dS0, ws, wsb, None)
        return L.osdn_gated_backward(B, 1, T, Dk, 32, 1, q, 0x20000, 0x30000,
                                     0x40000, None, 0.1, la, None, None, 1.0,
                                     0x60000, None, None, dq, 0x200000,
                                     0x300000, 0x400000, 0x500000, 0x600000,
                                     dla, 0x700000, dS0, ws, wsb, None)
    assert call(q=None) == NULL_ARG
    assert call(la=None) == NULL_ARG
    assert call(dla=None) == NULL_ARG
    assert call(dS0=None) == NULL_ARG
    assert call(T=-1) == BAD_DIMS
    assert call(Dk=16) == UNSUPPORTED
    assert call(ws=None) == WORKSPACE
    assert call(wsb=need - 4) == WORKSPACE
    assert call(ws=ws_at + 64) == WORKSPACE
    assert call(dq=0x10000 + 8) == ALIASING       # dq over q
    assert call(dla=0x80000) == ALIASING          # gradient over the decay
    assert call(dS0=ws_at) == ALIASING            # dS0 over the workspace
    assert call(B=0, q=None, la=None, dq=None, dS0=None, ws=None,
                dla=None) == OK
