"""The C ABI from plain C: tests/c/abi_host.c is compiled as C99 with
warnings as errors against include/psk_fused.h, linked against the built
library and run (host-side calls only, no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "elementwise_reduction_groups_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_program_uses_the_abi(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libpsk_fused.so")):
        pytest.skip("library not built")
    exe = str(tmp_path / "abi_host")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", LIBDIR, "-lpsk_fused",
                    "-Wl,-rpath," + LIBDIR, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
