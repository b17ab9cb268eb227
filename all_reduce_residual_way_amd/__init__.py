"""MI355X-native fused all-reduce + residual-add + RMSNorm epilogue (one GPU's share).

A thin ctypes binding over ``libfused_ar.so`` (built from ``csrc/`` by ``build.py``), with the
same entry points as the C ABI in ``include/fused_ar.h``. This module only marshals arguments:
every step of the operation runs in the library's HIP kernels. PyTorch supplies device memory and
streams. If the library is not built, every call raises; there is no fallback.

    from all_reduce_residual_way_amd import fused_ar_rmsnorm
    residual_out, out = fused_ar_rmsnorm(inputs, residual, weight, eps=1e-6)
"""
import contextlib
import ctypes
import os

__all__ = [
    "FusedArError", "Options", "library", "fused_ar_rmsnorm", "fused_ar_unfused_rmsnorm",
    "fused_ar_reduce", "fused_ar_rmsnorm_split", "split_workspace_bytes",
    "fused_ar_rmsnorm_split_ptrs", "fused_ar_rmsnorm_split_static",
    "fused_ar_rmsnorm_split_static_ptrs", "fused_ar_rmsnorm_ptrs", "fused_ar_rmsnorm_ex_ptrs",
    "fused_ar_unfused_rmsnorm_ptrs", "fused_ar_reduce_ptrs", "fused_ar_rmsnorm_check_ptrs",
    "auto_path", "auto_path_tp", "describe_launch", "strerror",
    "OK", "ERR_INVALID", "ERR_SHAPE", "ERR_ALIGN", "ERR_ALIAS", "ERR_SCRATCH",
    "STATIC_SCRATCH_FLOATS",
    "PATH_AUTO", "PATH_ONESTAGE", "PATH_TWOSTAGE", "PATH_UNFUSED", "WAVE_DPP", "WAVE_BPERMUTE",
    "STAGE1_FLAT", "STAGE1_LDS", "LOAD_AUTO", "LOAD_CACHED", "LOAD_STREAM", "CHUNKS_AUTO",
    "CHUNKS_SEQUENTIAL", "CHUNKS_PIPELINED", "RESIDUAL_AUTO", "RESIDUAL_STAGE2", "RESIDUAL_STAGE1",
    "MAX_INPUTS",
    "MAX_HIDDEN",
]

LIBRARY_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfused_ar.so")

# Values of include/fused_ar.h.
OK, ERR_INVALID, ERR_SHAPE, ERR_ALIGN, ERR_ALIAS, ERR_SCRATCH = 0, -1, -2, -3, -4, -5
PATH_AUTO, PATH_ONESTAGE, PATH_TWOSTAGE, PATH_UNFUSED = 0, 1, 2, 3
WAVE_DPP, WAVE_BPERMUTE = 0, 1
STAGE1_FLAT, STAGE1_LDS = 0, 1
LOAD_AUTO, LOAD_CACHED, LOAD_STREAM = 0, 1, 2
CHUNKS_AUTO, CHUNKS_SEQUENTIAL, CHUNKS_PIPELINED = 0, 1, 2
RESIDUAL_AUTO, RESIDUAL_STAGE2, RESIDUAL_STAGE1 = 0, 1, 2
MAX_INPUTS, MAX_HIDDEN = 8, 32768
STATIC_SCRATCH_FLOATS = 65536

_VP = ctypes.c_void_p


class _KernelLaunch(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("grid", ctypes.c_uint), ("block", ctypes.c_uint),
                ("per_thread", ctypes.c_uint), ("launches", ctypes.c_uint),
                ("streaming", ctypes.c_uint), ("lds_bytes", ctypes.c_uint)]


class _LaunchPlan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int), ("kernels", ctypes.c_int), ("launch", _KernelLaunch * 3)]


class Options(ctypes.Structure):
    """fused_ar_options: alternative kernel designs (see include/fused_ar.h)."""
    _fields_ = [("wave_reduce", ctypes.c_int), ("stage1", ctypes.c_int),
                ("stage1_block", ctypes.c_int), ("packs_per_thread", ctypes.c_int),
                ("load_policy", ctypes.c_int), ("stage_rows", ctypes.c_int),
                ("schedule", ctypes.c_int), ("residual_stage", ctypes.c_int)]


class FusedArError(RuntimeError):
    """A non-zero status from libfused_ar.so."""

    def __init__(self, status, what):
        super().__init__(f"{what}: status {status}: {strerror(status)}")
        self.status = status


_lib = None


def library():
    """The loaded ``libfused_ar.so`` (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise RuntimeError(
                f"{LIBRARY_PATH} is not built; build it with "
                "`python all_reduce_residual_way_amd/build.py`")
        # torch ships its own HIP runtime (same soname as ROCm's). Loading it first makes this
        # library bind to it; loaded the other way round, the process would hold two HIP and two
        # HSA runtimes, and the second to open the GPU finds no device.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIBRARY_PATH)
        lib.fused_ar_rmsnorm.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP, ctypes.c_float,
                                         ctypes.c_int, ctypes.c_int, _VP, _VP, ctypes.c_int, _VP]
        lib.fused_ar_rmsnorm.restype = ctypes.c_int
        lib.fused_ar_rmsnorm_ex.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP,
                                            ctypes.c_float, ctypes.c_int, ctypes.c_int, _VP, _VP,
                                            ctypes.c_int, ctypes.POINTER(Options), _VP]
        lib.fused_ar_rmsnorm_ex.restype = ctypes.c_int
        lib.fused_ar_unfused_rmsnorm.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP,
                                                 ctypes.c_float, ctypes.c_int, ctypes.c_int, _VP,
                                                 _VP, _VP]
        lib.fused_ar_unfused_rmsnorm.restype = ctypes.c_int
        lib.fused_ar_describe_launch_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int, ctypes.POINTER(Options),
                                                    ctypes.POINTER(_LaunchPlan)]
        lib.fused_ar_describe_launch_ex.restype = ctypes.c_int
        lib.fused_ar_rmsnorm_check.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP,
                                               ctypes.c_float, ctypes.c_int, ctypes.c_int, _VP,
                                               _VP, ctypes.c_int]
        lib.fused_ar_rmsnorm_check.restype = ctypes.c_int
        lib.fused_ar_reduce.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, _VP, _VP]
        lib.fused_ar_reduce.restype = ctypes.c_int
        lib.fused_ar_auto_path.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.fused_ar_auto_path.restype = ctypes.c_int
        lib.fused_ar_auto_path_tp.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.fused_ar_auto_path_tp.restype = ctypes.c_int
        lib.fused_ar_describe_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.POINTER(_LaunchPlan)]
        lib.fused_ar_describe_launch.restype = ctypes.c_int
        lib.fused_ar_rmsnorm_split.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP,
                                               ctypes.c_float, ctypes.c_int, ctypes.c_int, _VP,
                                               _VP, ctypes.c_int, _VP, ctypes.c_size_t, _VP]
        lib.fused_ar_rmsnorm_split.restype = ctypes.c_int
        lib.fused_ar_rmsnorm_split_static.argtypes = [ctypes.POINTER(_VP), ctypes.c_int, _VP, _VP,
                                                      ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                      _VP, _VP, ctypes.c_int, _VP]
        lib.fused_ar_rmsnorm_split_static.restype = ctypes.c_int
        lib.fused_ar_split_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.fused_ar_split_workspace_bytes.restype = ctypes.c_size_t
        lib.fused_ar_strerror.argtypes = [ctypes.c_int]
        lib.fused_ar_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def strerror(status):
    return library().fused_ar_strerror(int(status)).decode()


def auto_path(n, m, hidden):
    """The path (1 or 2) that ``path=0`` selects on one GPU; negative status for bad arguments."""
    return library().fused_ar_auto_path(int(n), int(m), int(hidden))


def auto_path_tp(n, m, hidden):
    """The pages' path rule for a tensor-parallel group over n GPUs (1 or 2); negative status for
    bad arguments."""
    return library().fused_ar_auto_path_tp(int(n), int(m), int(hidden))


def describe_launch(n, m, hidden, path=PATH_AUTO, options=None):
    """Kernels, grids and workgroup sizes of a call, as a dict; raises on bad arguments."""
    plan = _LaunchPlan()
    opt = ctypes.byref(options) if options is not None else None
    rc = library().fused_ar_describe_launch_ex(int(n), int(m), int(hidden), int(path), opt,
                                               ctypes.byref(plan))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_describe_launch")
    return {
        "path": plan.path,
        "kernels": [
            {"name": plan.launch[i].name.decode(), "grid": plan.launch[i].grid,
             "block": plan.launch[i].block, "per_thread": plan.launch[i].per_thread,
             "launches": plan.launch[i].launches, "streaming": plan.launch[i].streaming,
             "lds_bytes": plan.launch[i].lds_bytes}
            for i in range(plan.kernels)
        ],
    }


def _ptr_array(ptrs):
    return (_VP * len(ptrs))(*[int(p) for p in ptrs])


def fused_ar_rmsnorm_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out, out,
                          path=PATH_AUTO, stream=0):
    """Raw call with integer device addresses and a raw stream handle; returns the status."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_rmsnorm(arr, len(input_ptrs), _VP(residual), _VP(weight),
                                      float(eps), int(m), int(hidden), _VP(residual_out), _VP(out),
                                      int(path), _VP(stream))


def fused_ar_rmsnorm_ex_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out, out,
                             path=PATH_AUTO, options=None, stream=0):
    """Raw call of fused_ar_rmsnorm_ex; ``options`` is an Options or None; returns the status."""
    arr = _ptr_array(input_ptrs)
    opt = ctypes.byref(options) if options is not None else None
    return library().fused_ar_rmsnorm_ex(arr, len(input_ptrs), _VP(residual), _VP(weight),
                                         float(eps), int(m), int(hidden), _VP(residual_out),
                                         _VP(out), int(path), opt, _VP(stream))


def fused_ar_unfused_rmsnorm_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out,
                                  out, stream=0):
    """Raw call of the unfused three-kernel sequence; returns the status."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_unfused_rmsnorm(arr, len(input_ptrs), _VP(residual), _VP(weight),
                                              float(eps), int(m), int(hidden), _VP(residual_out),
                                              _VP(out), _VP(stream))


def fused_ar_rmsnorm_check_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out, out,
                                path=PATH_AUTO):
    """The status fused_ar_rmsnorm would return for these arguments, without launching."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_rmsnorm_check(arr, len(input_ptrs), _VP(residual), _VP(weight),
                                            float(eps), int(m), int(hidden), _VP(residual_out),
                                            _VP(out), int(path))


def fused_ar_reduce_ptrs(input_ptrs, m, hidden, reduced, stream=0):
    """Raw call of the reduce alone; returns the status."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_reduce(arr, len(input_ptrs), int(m), int(hidden), _VP(reduced),
                                     _VP(stream))


def split_workspace_bytes(m, hidden, splits=0):
    """Workspace bytes fused_ar_rmsnorm_split needs (0 for m == 0 or invalid scalars)."""
    return int(library().fused_ar_split_workspace_bytes(int(m), int(hidden), int(splits)))


def fused_ar_rmsnorm_split_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out, out,
                                splits, workspace, workspace_bytes, stream=0):
    """Raw call of the split-row form; returns the status."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_rmsnorm_split(arr, len(input_ptrs), _VP(residual), _VP(weight),
                                            float(eps), int(m), int(hidden), _VP(residual_out),
                                            _VP(out), int(splits), _VP(workspace),
                                            int(workspace_bytes), _VP(stream))


def fused_ar_rmsnorm_split_static_ptrs(input_ptrs, residual, weight, eps, m, hidden, residual_out,
                                       out, splits=0, stream=0):
    """Raw call of the split-row form that allocates nothing (its slice square-sums in the
    library's static scratch); returns the status."""
    arr = _ptr_array(input_ptrs)
    return library().fused_ar_rmsnorm_split_static(arr, len(input_ptrs), _VP(residual),
                                                   _VP(weight), float(eps), int(m), int(hidden),
                                                   _VP(residual_out), _VP(out), int(splits),
                                                   _VP(stream))


_torch = None


def _torch_module():
    global _torch
    if _torch is None:
        import torch
        _torch = torch
    return _torch


def _check_tensor(t, name, shape, device):
    """Raise the error that describes why ``t`` is not a contiguous bf16 tensor of ``shape`` on
    ``device`` (nothing if it is one)."""
    torch = _torch_module()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device or 'a GPU'}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fits(t, shape, index, torch):
    """True if ``t`` is a contiguous bf16 CUDA tensor of ``shape`` on device ``index`` (the cheap
    test made on every call; _check_tensor explains a failure)."""
    return (isinstance(t, torch.Tensor) and t.dtype is torch.bfloat16 and t.shape == shape
            and t.get_device() == index and t.is_contiguous())


_NO_GUARD = contextlib.nullcontext()


def _device_guard(device):
    """Makes ``device`` the current device for the call (the library launches on the current
    device, and the default stream handle 0 means that device's null stream); no-op if it is."""
    torch = _torch_module()
    if device.index == torch.cuda.current_device():
        return _NO_GUARD
    return torch.cuda.device(device.index)


def _stream_handle(stream, device):
    torch = _torch_module()
    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)  # no Stream object per call
    if raw is not None:
        return raw(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _check_stream(stream, device):
    """Raise unless ``stream`` (a torch.cuda.Stream, or None for the current stream) belongs to
    ``device``, the device of the tensors: the kernels run on the device the stream belongs to."""
    if stream is not None and stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")


def _on_stream(t, stream):
    """A tensor allocated here for work enqueued on ``stream`` (not the current stream): recorded
    on that stream, so that torch's caching allocator does not hand its memory out again before
    that work is done, even if the caller drops the tensor at once."""
    if stream is not None:
        t.record_stream(stream)
    return t


def _prepare(inputs, residual, weight, residual_out, out, stream=None):
    torch = _torch_module()
    if not isinstance(inputs, (list, tuple)) or not inputs:
        raise ValueError("inputs must be a non-empty list of tensors")
    if not isinstance(residual, torch.Tensor) or residual.dim() != 2:
        raise ValueError("residual must be a 2-D tensor (m, hidden)")
    shape = residual.shape
    m, hidden = shape
    device = residual.device
    _check_stream(stream, device)
    index = device.index if device.type == "cuda" else -2  # get_device() is -1 on the CPU
    if not (all(_fits(x, shape, index, torch) for x in inputs)
            and _fits(residual, shape, index, torch) and _fits(weight, (hidden,), index, torch)):
        for i, x in enumerate(inputs):
            _check_tensor(x, f"inputs[{i}]", (m, hidden), device)
        _check_tensor(residual, "residual", (m, hidden), device)
        _check_tensor(weight, "weight", (hidden,), device)
    if residual_out is None:
        residual_out = _on_stream(torch.empty_like(residual), stream)
    elif not _fits(residual_out, shape, index, torch):
        _check_tensor(residual_out, "residual_out", (m, hidden), device)
    if out is None:
        out = _on_stream(torch.empty_like(residual), stream)
    elif not _fits(out, shape, index, torch):
        _check_tensor(out, "out", (m, hidden), device)
    return m, hidden, device, residual_out, out


def fused_ar_rmsnorm(inputs, residual, weight, eps=1e-6, *, residual_out=None, out=None,
                     path=PATH_AUTO, stream=None, options=None):
    """The fused epilogue on one GPU.

    Args:
        inputs: list of n (1..8) bf16 CUDA tensors of shape (m, hidden), the partial sums; they
            are reduced in fp32 in list order.
        residual: bf16 (m, hidden). weight: bf16 (hidden,). eps: float >= 0.
        residual_out: optional bf16 (m, hidden) output buffer; may be ``residual`` itself.
        out: optional bf16 (m, hidden) output buffer, overlapping nothing else (the two-stage path
            also uses it as scratch).
        path: 0 automatic, 1 one-stage, 2 two-stage (3: the unfused three-kernel sequence).
        stream: torch.cuda.Stream to enqueue on (default: the current stream).
        options: an Options (alternative kernel designs) or None for the defaults.
    Returns:
        (residual_out, out). Missing outputs are allocated with ``torch.empty_like(residual)``
        (recorded on ``stream`` when one is given) and belong to the caller. The work is
        asynchronous on the stream.
    Raises:
        TypeError/ValueError for tensors of the wrong dtype, device, shape or layout;
        FusedArError for a non-zero library status.
    """
    m, hidden, device, residual_out, out = _prepare(inputs, residual, weight, residual_out, out,
                                                    stream)
    n = len(inputs)
    arr = (_VP * n)(*[x.data_ptr() for x in inputs])
    with _device_guard(device):
        rc = library().fused_ar_rmsnorm_ex(arr, n, residual.data_ptr(), weight.data_ptr(), eps, m,
                                           hidden, residual_out.data_ptr(), out.data_ptr(), path,
                                           None if options is None else ctypes.byref(options),
                                           _stream_handle(stream, device))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_rmsnorm")
    return residual_out, out


def fused_ar_unfused_rmsnorm(inputs, residual, weight, eps=1e-6, *, residual_out=None, out=None,
                             stream=None):
    """The same result as fused_ar_rmsnorm, computed as three kernels (reduce, residual add,
    RMSNorm): the unfused baseline. Arguments and returns as fused_ar_rmsnorm (no path)."""
    m, hidden, device, residual_out, out = _prepare(inputs, residual, weight, residual_out, out,
                                                    stream)
    with _device_guard(device):
        rc = fused_ar_unfused_rmsnorm_ptrs([x.data_ptr() for x in inputs], residual.data_ptr(),
                                           weight.data_ptr(), eps, m, hidden,
                                           residual_out.data_ptr(), out.data_ptr(),
                                           _stream_handle(stream, device))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_unfused_rmsnorm")
    return residual_out, out


def fused_ar_reduce(inputs, *, reduced=None, stream=None):
    """The N-way reduce alone (the two-stage path's first kernel): bf16 of the fp32 sum of
    ``inputs`` (list of bf16 (m, hidden) CUDA tensors) in list order. Returns ``reduced``."""
    import torch
    if not isinstance(inputs, (list, tuple)) or not inputs:
        raise ValueError("inputs must be a non-empty list of tensors")
    x0 = inputs[0]
    if not isinstance(x0, torch.Tensor) or x0.dim() != 2:
        raise ValueError("inputs must be 2-D tensors (m, hidden)")
    m, hidden = x0.shape
    for i, x in enumerate(inputs):
        _check_tensor(x, f"inputs[{i}]", (m, hidden), x0.device)
    _check_stream(stream, x0.device)
    if reduced is None:
        reduced = _on_stream(torch.empty_like(x0), stream)
    _check_tensor(reduced, "reduced", (m, hidden), x0.device)
    with _device_guard(x0.device):
        rc = fused_ar_reduce_ptrs([x.data_ptr() for x in inputs], m, hidden, reduced.data_ptr(),
                                  _stream_handle(stream, x0.device))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_reduce")
    return reduced


def fused_ar_rmsnorm_split(inputs, residual, weight, eps=1e-6, *, splits=0, workspace=None,
                           residual_out=None, out=None, stream=None):
    """The one-stage result with each row cut into ``splits`` slices on separate workgroups (0 =
    one slice per 256 packs), in two kernels. ``workspace`` is a CUDA tensor of at least
    ``split_workspace_bytes(m, hidden, splits)`` bytes, allocated here when None. Other arguments
    and returns as fused_ar_rmsnorm (always the one-stage path)."""
    import torch
    m, hidden, device, residual_out, out = _prepare(inputs, residual, weight, residual_out, out,
                                                    stream)
    need = split_workspace_bytes(m, hidden, splits)
    if workspace is None:
        workspace = _on_stream(torch.empty(max(need, 4) // 4, dtype=torch.float32, device=device),
                               stream)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device:
        raise ValueError(f"workspace must be a tensor on {device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    with _device_guard(device):
        rc = fused_ar_rmsnorm_split_ptrs([x.data_ptr() for x in inputs], residual.data_ptr(),
                                         weight.data_ptr(), eps, m, hidden,
                                         residual_out.data_ptr(), out.data_ptr(), splits,
                                         workspace.data_ptr(), nbytes,
                                         _stream_handle(stream, device))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_rmsnorm_split")
    return residual_out, out


def fused_ar_rmsnorm_split_static(inputs, residual, weight, eps=1e-6, *, splits=0,
                                  residual_out=None, out=None, stream=None):
    """fused_ar_rmsnorm_split with the slice square-sums in the library's static scratch instead of
    a workspace: the library call allocates nothing (for callers that cannot allocate, e.g. under
    graph capture; pass both outputs to allocate nothing here either). At most
    STATIC_SCRATCH_FLOATS slice square-sums (m * slices) per call; calls on one GPU must not
    overlap in time (they share the scratch). Other arguments and returns as
    fused_ar_rmsnorm_split."""
    m, hidden, device, residual_out, out = _prepare(inputs, residual, weight, residual_out, out,
                                                    stream)
    n = len(inputs)
    arr = (_VP * n)(*[x.data_ptr() for x in inputs])
    with _device_guard(device):
        rc = library().fused_ar_rmsnorm_split_static(arr, n, residual.data_ptr(),
                                                     weight.data_ptr(), eps, m, hidden,
                                                     residual_out.data_ptr(), out.data_ptr(),
                                                     int(splits), _stream_handle(stream, device))
    if rc != OK:
        raise FusedArError(rc, "fused_ar_rmsnorm_split_static")
    return residual_out, out
