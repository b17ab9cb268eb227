"""CPU oracle for the fused all-reduce + residual + RMSNorm epilogue.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The HIP path never calls it and shares no
code with it.

The arithmetic lives in ``fused_ar_oracle.c`` (plain single-threaded C, strict IEEE); this module
only marshals numpy arrays of raw bf16 bit patterns (``uint16``) into it. What it computes, and
which passage of the pages each step follows, is stated at the top of that file.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_U16P = ctypes.POINTER(ctypes.c_uint16)


def _ptr(a):
    return a.ctypes.data_as(_U16P)


def _as_bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected raw bf16 bits as uint16, got {a.dtype}")
    return a


class Oracle:
    """One loaded copy of the oracle library (the default one, or a test build of it)."""

    def __init__(self, library=None):
        if library is None:
            library = _build.LIBRARY
            if not os.path.exists(library):
                _build.build()
        self.path = library
        lib = ctypes.CDLL(library)
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_reduce.argtypes = [ctypes.POINTER(_U16P), ctypes.c_int, ctypes.c_longlong, _U16P]
        lib.oracle_reduce.restype = ctypes.c_int
        lib.oracle_fused_ar_rmsnorm.argtypes = [
            ctypes.POINTER(_U16P), ctypes.c_int, _U16P, _U16P, ctypes.c_float, ctypes.c_int,
            ctypes.c_int, _U16P, _U16P]
        lib.oracle_fused_ar_rmsnorm.restype = ctypes.c_int
        self._lib = lib

    def bf16_round(self, x):
        """Bits of the bf16 nearest to the real ``x`` (ties to even)."""
        return int(self._lib.oracle_bf16_round(float(x)))

    def reduce(self, inputs):
        """Elementwise fp32 sum of ``inputs`` (list of same-shape uint16 arrays) in list order, as bf16 bits."""
        ins = [_as_bits(a) for a in inputs]
        shape = ins[0].shape
        if any(a.shape != shape for a in ins):
            raise ValueError("inputs differ in shape")
        arr = (_U16P * len(ins))(*[_ptr(a) for a in ins])
        red = np.empty(shape, dtype=np.uint16)
        rc = self._lib.oracle_reduce(arr, len(ins), int(red.size), _ptr(red))
        if rc != 0:
            raise ValueError("oracle_reduce rejected its arguments")
        return red

    def fused(self, inputs, residual, weight, eps):
        """(residual_out, out) for inputs [n x (m, hidden)], residual (m, hidden), weight (hidden,)."""
        ins = [_as_bits(a) for a in inputs]
        residual = _as_bits(residual)
        weight = _as_bits(weight)
        m, hidden = residual.shape
        if any(a.shape != (m, hidden) for a in ins) or weight.shape != (hidden,):
            raise ValueError("shape mismatch")
        ro = np.empty((m, hidden), dtype=np.uint16)
        out = np.empty((m, hidden), dtype=np.uint16)
        self._fused_into(ins, residual, weight, eps, ro, out)
        return ro, out

    def _fused_into(self, ins, residual, weight, eps, ro, out):
        m, hidden = residual.shape
        arr = (_U16P * len(ins))(*[_ptr(a) for a in ins])
        rc = self._lib.oracle_fused_ar_rmsnorm(arr, len(ins), _ptr(residual), _ptr(weight),
                                               float(eps), m, hidden, _ptr(ro), _ptr(out))
        if rc != 0:
            raise ValueError("oracle_fused_ar_rmsnorm rejected its arguments")

    def fused_threads(self, inputs, residual, weight, eps, threads):
        """``fused`` with the rows cut into ``threads`` contiguous slices, each slice computed by the
        same single-threaded C function on its own host thread (ctypes releases the GIL during the
        call). Rows are independent in the oracle, so the result is the same bits as ``fused``."""
        import concurrent.futures as cf
        ins = [_as_bits(a) for a in inputs]
        residual = _as_bits(residual)
        weight = _as_bits(weight)
        m, hidden = residual.shape
        if any(a.shape != (m, hidden) for a in ins) or weight.shape != (hidden,):
            raise ValueError("shape mismatch")
        ro = np.empty((m, hidden), dtype=np.uint16)
        out = np.empty((m, hidden), dtype=np.uint16)
        threads = max(1, min(int(threads), m))
        bounds = [(m * t // threads, m * (t + 1) // threads) for t in range(threads)]
        bounds = [(a, b) for a, b in bounds if b > a]

        def piece(ab):
            a, b = ab
            self._fused_into([x[a:b] for x in ins], residual[a:b], weight, eps, ro[a:b], out[a:b])

        with cf.ThreadPoolExecutor(max(1, len(bounds))) as pool:
            list(pool.map(piece, bounds))
        return ro, out


_default = None


def default():
    """The oracle built from ``fused_ar_oracle.c`` in this directory (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def bf16_round(x):
    return default().bf16_round(x)


def reduce(inputs):
    return default().reduce(inputs)


def fused(inputs, residual, weight, eps):
    return default().fused(inputs, residual, weight, eps)


def fused_threads(inputs, residual, weight, eps, threads):
    return default().fused_threads(inputs, residual, weight, eps, threads)
