"""The host library under AddressSanitizer (CPU only): the host sources
(validator, emitter, hipRTC driver, partition, C ABI) are compiled with g++
and -fsanitize=address, linked with the gfx950 kernel object of the normal
build and with the plain-C ABI program tests/c/abi_host.c, and run; any
out-of-bounds access or use after free in the host paths fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "elementwise_reduction_groups_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _has_asan():
    if shutil.which("g++") is None:
        return False
    r = subprocess.run(["g++", "-fsanitize=address", "-x", "c++", "-", "-o", os.devnull],
                       input="int main(){return 0;}", capture_output=True, text=True)
    return r.returncode == 0


@pytest.mark.skipif(not _has_asan(), reason="no g++ with AddressSanitizer")
def test_host_paths_under_address_sanitizer(tmp_path):
    from elementwise_reduction_groups_amd import build as B
    kernel_obj = os.path.join(B.BUILD, "adamw.hip.o")
    if not os.path.exists(kernel_obj):
        pytest.skip("library not built")
    objs = []
    for s in B.HOST_SOURCES:
        o = str(tmp_path / (s + ".o"))
        subprocess.run(["g++", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
                        f"-I{B.INCLUDE}", f"-I{B.CSRC}", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-c",
                        os.path.join(B.CSRC, s), "-o", o], check=True)
        objs.append(o)
    main_obj = str(tmp_path / "abi_host.o")
    subprocess.run(["gcc", "-std=c99", "-g", "-fsanitize=address", f"-I{B.INCLUDE}", "-c",
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", main_obj], check=True)
    exe = str(tmp_path / "abi_host_asan")
    subprocess.run(["g++", "-fsanitize=address", main_obj, *objs, kernel_obj, f"-L{ROCM}/lib", "-lamdhip64", "-lhiprtc",
                    f"-Wl,-rpath,{ROCM}/lib", "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-3000:] + r.stderr[-6000:]
