"""Build libfused_ar.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "fused_ar.hip")]
LIBRARY = os.path.join(PKG, "libfused_ar.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # binary32 subnormals are kept, as IEEE arithmetic requires
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wextra", "-Wno-unused-command-line-argument",
]


def hipcc():
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError(f"hipcc not found (looked for {path})")
    return path


def build(output=LIBRARY, extra_flags=(), verbose=False, sources=SOURCES):
    """Compile the HIP ``sources`` into ``output``; returns its path. Always recompiles."""
    tmp = output + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
