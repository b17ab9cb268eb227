"""The benchmark's HBM ceiling probes (libhbm_probe.so, built from hbm_probe.hip by build.py):
plain streaming kernels for a read stream, a copy, the one-stage kernel's nine-read /
two-write mix, mixes of 5 or 9 reads with 1 or 2 writes, and a mix's reads alone and its writes
alone. Measurement infrastructure for bench.py --ceilings and its test; the fused path
does not use it."""
import ctypes
import os

from . import build as _build

LIBRARY = _build.LIBRARY


def load():
    """The loaded probe library with its argument types set; raises if it is not built."""
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is not built; build it with `python hbm_probe/build.py`")
    import torch  # noqa: F401  (bind to torch's HIP runtime, as the fused library does)
    vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib = ctypes.CDLL(LIBRARY)
    lib.hbm_probe_read.argtypes = [vp, sz, vp, ci, ci, ci, vp]
    lib.hbm_probe_copy.argtypes = [vp, vp, sz, ci, ci, vp]
    lib.hbm_probe_mix.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), sz, ci, ci, vp]
    lib.hbm_probe_mix_rw.argtypes = [ctypes.POINTER(vp), ci, ctypes.POINTER(vp), ci, sz, ci, ci, vp]
    lib.hbm_probe_reads.argtypes = [ctypes.POINTER(vp), ci, sz, vp, ci, ci, vp]
    lib.hbm_probe_writes.argtypes = [ctypes.POINTER(vp), ci, sz, ci, ci, vp]
    return lib
