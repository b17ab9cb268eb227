"""The library's host code (argument checks, launch plans) under AddressSanitizer and
UndefinedBehaviorSanitizer: the HIP source is rebuilt with the sanitizers on the host pass only
(-Xarch_host; device code is unchanged) and the C client's CPU mode drives every entry point that
needs no GPU, including the extreme scalar arguments. Any sanitizer report fails the test."""
import os
import subprocess

import pytest

from all_reduce_residual_way_amd import build as hip_build
from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(oracle_build.LIBRARY):
        oracle_build.build()
    lib = str(tmp_path / "libfused_ar_sanitized.so")
    host_flags = []
    for f in SANITIZE:
        host_flags += ["-Xarch_host", f]
    flags = [f for f in hip_build.FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([hip_build.hipcc(), *flags, *host_flags, "-I", hip_build.INCLUDE,
                    "-I", hip_build.CSRC, "-o", lib, *hip_build.SOURCES], check=True,
                   stderr=subprocess.DEVNULL)
    exe = str(tmp_path / "fused_ar_c_check")
    subprocess.run([CLANG, "-std=c11", "-g", *SANITIZE, "-D__HIP_PLATFORM_AMD__",
                    "-I", hip_build.INCLUDE, "-I", os.path.join(ROCM, "include"),
                    os.path.join(HERE, "c_abi", "fused_ar_c_check.c"), "-o", exe, lib,
                    oracle_build.LIBRARY, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    f"-Wl,-rpath,{tmp_path}:{os.path.dirname(oracle_build.LIBRARY)}:"
                    f"{os.path.join(ROCM, 'lib')}"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe, "cpu"], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert "cpu checks passed" in r.stdout
