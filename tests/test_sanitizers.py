"""The library's host code under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU: osdn_api.cpp, ktimer.cpp and the host side of
noalloc.hip are rebuilt with the sanitizers (host code only; the device code
objects of the regular in-tree build are linked unchanged), and the plain C
consumer (tests/c/abi_consumer.c), built with the same sanitizers, drives
every host-side path it covers: capability and workspace queries for every
entry point, argument validation, aliasing checks, the allocation-free
entry point's size check and the kernel-timing record. Any sanitizer report
fails the test. No GPU is used."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "delta_rule_recurrent_scan_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HOST_SOURCES = ("osdn_api.cpp", "ktimer.cpp", "noalloc.hip")


def _device_objects():
    return [o for o in glob.glob(os.path.join(BUILD, "*.o"))
            if os.path.basename(o)[:-2] not in HOST_SOURCES]


def _runtime_dir():
    d = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux")
    return d[0] if d else None


needs_toolchain = pytest.mark.skipif(
    not (os.path.exists(HIPCC) and os.path.exists(CLANG) and _runtime_dir()),
    reason="ROCm clang toolchain with sanitizer runtimes not found")
needs_build = pytest.mark.skipif(
    len(_device_objects()) < 5, reason="in-tree build objects (_build/) missing")


@needs_toolchain
@needs_build
def test_host_code_under_asan_and_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-fno-omit-frame-pointer"]
    objs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-I",
               os.path.join(ROOT, "include")] + san
        if src.endswith(".hip"):
            cmd += ["-x", "hip", "--offload-arch=gfx950", "-Xclang",
                    "-target-feature", "-Xclang", "-packed-fp32-ops"]
        subprocess.run(cmd + ["-c", os.path.join(CSRC, src), "-o", obj],
                       check=True, capture_output=True)
        objs.append(obj)
    rt = _runtime_dir()
    lib = str(tmp_path / "libosdn_san.so")
    subprocess.run([CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-shared-libsan", "-o", lib] + objs + _device_objects()
                   + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                      "-Wl,-rpath," + rt], check=True, capture_output=True)
    exe = str(tmp_path / "abi_consumer_san")
    subprocess.run([CLANG, "-std=c99", "-Wall", "-Werror", "-O1", "-g",
                    "-fsanitize=address,undefined", "-shared-libsan",
                    "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", exe,
                    "-L", str(tmp_path), "-losdn_san",
                    "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt],
                   check=True, capture_output=True)
    env = dict(os.environ,
               ASAN_OPTIONS="halt_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out
    assert "all checks passed" in p.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
