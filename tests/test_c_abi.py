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


def _build_gpu_program(tmp_path) -> str:
    """tests/c/abi_gpu.c as C99, warnings as errors, against the library, the
    HIP runtime's C API and the C oracle (which only tests link)."""
    for lib in [os.path.join(LIBDIR, "libpsk_fused.so"), os.path.join(ROOT, "oracle", "liboracle.so")]:
        if not os.path.exists(lib):
            pytest.skip(f"{os.path.basename(lib)} not built")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "abi_gpu")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(rocm, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_gpu.c"),
                    "-L", LIBDIR, "-lpsk_fused", "-L", os.path.join(ROOT, "oracle"), "-loracle",
                    "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
                    "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROOT, "oracle"),
                    "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe], check=True)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_gpu_program_builds(tmp_path):
    assert os.path.exists(_build_gpu_program(tmp_path))


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_gpu_program_runs_against_the_oracle(tmp_path):
    """Softmax (register and tiled kernels) and an AdamW step from plain C on
    the GPU, checked inside the program against the C oracle."""
    exe = _build_gpu_program(tmp_path)
    print("running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
