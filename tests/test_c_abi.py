"""A plain C11 client of the library (tests/c_abi/fused_ar_c_check.c), built with gcc against
include/fused_ar.h only: the boundary is usable as a C ABI without Python or C++."""
import os
import subprocess

import pytest

import all_reduce_residual_way_amd as fa
from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "c_abi", "fused_ar_c_check.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    fa.library()  # the product library must be built
    if not os.path.exists(oracle_build.LIBRARY):
        oracle_build.build()
    exe = str(tmp_path_factory.mktemp("c_abi") / "fused_ar_c_check")
    libdir = os.path.dirname(fa.LIBRARY_PATH)
    odir = os.path.dirname(oracle_build.LIBRARY)
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SOURCE,
           "-o", exe, fa.LIBRARY_PATH, oracle_build.LIBRARY,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}:{odir}:{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True)
    return exe


def test_c_client_cpu_entry_points(program):
    r = subprocess.run([program, "cpu"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "cpu checks passed" in r.stdout


@pytest.mark.gpu
def test_c_client_on_gpu(program):
    print("[gpu case] C client, n=5 m=7 hidden=520, paths 1, 2, unfused, graph capture, split rows, reduce", flush=True)
    r = subprocess.run([program, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "gpu checks passed" in r.stdout
