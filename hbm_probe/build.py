"""Build libhbm_probe.so (the benchmark's HBM ceiling probes) for gfx950 with hipcc, in-tree.

Measurement infrastructure beside bench.py: the fused path neither builds nor loads it."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "hbm_probe.hip")]
LIBRARY = os.path.join(HERE, "libhbm_probe.so")


def build(verbose=False):
    """Compile the probes into libhbm_probe.so with the library's flags; returns its path."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from all_reduce_residual_way_amd import build as hip_build
    return hip_build.build(LIBRARY, verbose=verbose, sources=SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
