"""The C ABI used from plain C: tests/c/abi_consumer.c is compiled with the
system C compiler against include/osdn.h, linked with libosdn.so and run.
It exercises only host-side paths (queries and argument validation), so it
needs no GPU."""
import os
import shutil
import subprocess

import pytest

import delta_rule_recurrent_scan_amd as osdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = osdn.library_path()


@pytest.mark.skipif(not os.path.exists(LIB), reason="libosdn.so not built")
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_consumer(tmp_path):
    exe = tmp_path / "abi_consumer"
    libdir = os.path.dirname(LIB)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_consumer.c"),
                    "-L", libdir, "-losdn", "-Wl,-rpath," + libdir,
                    "-o", str(exe)], check=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "all checks passed" in p.stdout
