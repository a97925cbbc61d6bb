"""MI355X-native FNO spectral convolution: Python binding of libfno.so.

The functions mirror the C ABI in include/fno.h one to one and only marshal
arguments (torch tensors -> device pointers, the current HIP stream); every
step of the layer runs in the library's HIP kernels. There is no CPU path:
if libfno.so is missing, importing a function that needs it raises.
"""

import ctypes

from ._lib import DTYPES, FnoError, check, lib  # noqa: F401

__all__ = [
    "fno_plan_create", "fno_spectral_conv2d", "fno_spectral_conv3d",
    "fno_plan_destroy", "fno_status_string", "fno_plan_workspace_bytes",
    "fno_plan_num_launches", "fno_plan_launch_name", "fno_plan_run_launch",
    "fno_plan_spectra", "SpectralConv", "FnoError", "DTYPES",
]


def _torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream, device):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream(device).cuda_stream


class Plan:
    """Handle of a C plan plus the shape it was made for."""

    def __init__(self, handle, ndim, batch, c_in, c_out, grid, modes, dtype, device):
        self.handle = handle
        self.ndim, self.batch, self.c_in, self.c_out = ndim, batch, c_in, c_out
        self.grid, self.modes, self.dtype, self.device = tuple(grid), tuple(modes), dtype, device

    @property
    def n_modes(self):
        k = 1
        for m in self.modes:
            k *= m
        return k * (2 if self.ndim == 2 else 4)

    def x_shape(self):
        return (self.batch, self.c_in) + self.grid

    def y_shape(self):
        return (self.batch, self.c_out) + self.grid

    def w_shape(self):
        if self.ndim == 2:
            return (2 * self.modes[0], self.modes[1], self.c_in, self.c_out, 2)
        return (2 * self.modes[0], 2 * self.modes[1], self.modes[2], self.c_in, self.c_out, 2)


def fno_status_string(status):
    return lib().fno_status_string(status).decode()


def fno_plan_create(ndim, batch, c_in, c_out, grid, modes, dtype="f32", device=0):
    """Make a plan (see fno_plan_create in include/fno.h). Returns a Plan."""
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {list(DTYPES)}")
    h = ctypes.c_void_p()
    g = (ctypes.c_int * len(grid))(*grid)
    m = (ctypes.c_int * len(modes))(*modes)
    check(lib().fno_plan_create(ctypes.byref(h), ndim, batch, c_in, c_out, g, m,
                                DTYPES[dtype], device), "fno_plan_create")
    return Plan(h, ndim, batch, c_in, c_out, grid, modes, dtype, device)


def _check_tensors(plan, x, w, y):
    import torch
    if isinstance(x, int) or isinstance(w, int) or isinstance(y, int):
        return
    td = _torch_dtype(plan.dtype)
    for name, t, shape in (("x", x, plan.x_shape()), ("w", w, plan.w_shape()),
                           ("y", y, plan.y_shape())):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor or a device pointer")
        if t.dtype != td:
            raise ValueError(f"{name} dtype {t.dtype} != plan dtype {td}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")


def fno_spectral_conv2d(plan, x, w, y, stream=None):
    _check_tensors(plan, x, w, y)
    check(lib().fno_spectral_conv2d(plan.handle, _ptr(x), _ptr(w), _ptr(y),
                                    _stream(stream, plan.device)), "fno_spectral_conv2d")


def fno_spectral_conv3d(plan, x, w, y, stream=None):
    _check_tensors(plan, x, w, y)
    check(lib().fno_spectral_conv3d(plan.handle, _ptr(x), _ptr(w), _ptr(y),
                                    _stream(stream, plan.device)), "fno_spectral_conv3d")


def fno_plan_destroy(plan):
    if plan is None or plan.handle is None:
        return
    check(lib().fno_plan_destroy(plan.handle), "fno_plan_destroy")
    plan.handle = None


def fno_plan_workspace_bytes(plan):
    n = ctypes.c_size_t()
    check(lib().fno_plan_workspace_bytes(plan.handle, ctypes.byref(n)), "fno_plan_workspace_bytes")
    return n.value


def fno_plan_num_launches(plan):
    n = ctypes.c_int()
    check(lib().fno_plan_num_launches(plan.handle, ctypes.byref(n)), "fno_plan_num_launches")
    return n.value


def fno_plan_launch_name(plan, index):
    s = ctypes.c_char_p()
    check(lib().fno_plan_launch_name(plan.handle, index, ctypes.byref(s)), "fno_plan_launch_name")
    return s.value.decode()


def fno_plan_run_launch(plan, index, x, w, y, stream=None):
    _check_tensors(plan, x, w, y)
    check(lib().fno_plan_run_launch(plan.handle, index, _ptr(x), _ptr(w), _ptr(y),
                                    _stream(stream, plan.device)), "fno_plan_run_launch")


def fno_plan_spectra(plan, which):
    """Device pointer of the forward (0) or contracted (1) spectra workspace."""
    p = ctypes.c_void_p()
    check(lib().fno_plan_spectra(plan.handle, which, ctypes.byref(p)), "fno_plan_spectra")
    return p.value


class SpectralConv:
    """Owns a plan; call with (x, w[, y]) torch tensors on the plan's device."""

    def __init__(self, ndim, batch, c_in, c_out, grid, modes, dtype="f32", device=0):
        self.plan = fno_plan_create(ndim, batch, c_in, c_out, grid, modes, dtype, device)

    def __call__(self, x, w, y=None, stream=None):
        import torch
        if y is None:
            y = torch.empty(self.plan.y_shape(), dtype=_torch_dtype(self.plan.dtype),
                            device=x.device)
        f = fno_spectral_conv2d if self.plan.ndim == 2 else fno_spectral_conv3d
        f(self.plan, x, w, y, stream)
        return y

    def close(self):
        fno_plan_destroy(self.plan)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
