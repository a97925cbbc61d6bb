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
    "fno_plan_spectra", "fno_spectral_conv2d_backward", "fno_spectral_conv3d_backward", "SpectralConv", "FnoError", "DTYPES",
    "fno_weights_pack", "fno_weights_unpack", "SpectralConvFunction", "spectral_conv",
    "fno_channel_mix", "fno_projection", "fno_model2d_create", "fno_model2d_forward",
    "fno_model2d_destroy", "Model2d", "fno_model2d_set_graph", "fno_block2d", "fno_block2d_prepare",
    "fno_plan_saved_bytes", "fno_saved_empty", "fno_spectral_conv_forward_save",
    "fno_spectral_conv_backward_saved",
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

    def split_shape(self):
        """Shape of each of weight_real / weight_imag (modes first)."""
        return self.w_shape()[:-1]

    def corners_shape(self):
        """Shape of the stacked per-corner weights, channels first, (re, im) last."""
        return (2 if self.ndim == 2 else 4, self.c_in, self.c_out) + self.modes + (2,)


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


def fno_spectral_conv_noalloc(plan, x, w, y, stream=None):
    """The layer (2D or 3D as the plan says) with its exchange buffers in
    the library's static scratch array instead of the plan's workspace; see
    fno_spectral_conv_noalloc in include/fno.h."""
    _check_tensors(plan, x, w, y)
    check(lib().fno_spectral_conv_noalloc(plan.handle, _ptr(x), _ptr(w), _ptr(y),
                                          _stream(stream, plan.device)), "fno_spectral_conv_noalloc")


def fno_block2d(plan, x, w, bypass, bias, y, act=1, stream=None):
    """One FNO block, y = act(spectral conv(x, w) + bypass x + bias), with the
    spectral branch finished in the epilogue; see fno_block2d in
    include/fno.h. bypass [c_out][c_in], bias [c_out] or None."""
    _check_tensors(plan, x, w, y)
    check(lib().fno_block2d(plan.handle, _ptr(x), _ptr(w), _ptr(bypass), _ptr(bias), act, _ptr(y),
                            _stream(stream, plan.device)), "fno_block2d")


def fno_block2d_prepare(plan):
    """Allocate the plan's block buffer now (before a graph capture)."""
    check(lib().fno_block2d_prepare(plan.handle), "fno_block2d_prepare")


def _check_backward(plan, x, w, gy, gx, gw):
    import torch
    td = _torch_dtype(plan.dtype)
    for name, t, shape in (("x", x, plan.x_shape()), ("w", w, plan.w_shape()),
                           ("grad_y", gy, plan.y_shape()), ("grad_x", gx, plan.x_shape()),
                           ("grad_w", gw, plan.w_shape())):
        if t is None or isinstance(t, int):
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor, a device pointer or None")
        if t.dtype != td:
            raise ValueError(f"{name} dtype {t.dtype} != plan dtype {td}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")


def fno_spectral_conv2d_backward(plan, x, w, grad_y, grad_x, grad_w, stream=None):
    """Gradients of the 2D layer (see include/fno.h); grad_x or grad_w may be None."""
    _check_backward(plan, x, w, grad_y, grad_x, grad_w)
    check(lib().fno_spectral_conv2d_backward(plan.handle, _ptr(x), _ptr(w), _ptr(grad_y), _ptr(grad_x),
                                             _ptr(grad_w), _stream(stream, plan.device)),
          "fno_spectral_conv2d_backward")


def fno_spectral_conv3d_backward(plan, x, w, grad_y, grad_x, grad_w, stream=None):
    """Gradients of the 3D layer; as fno_spectral_conv2d_backward."""
    _check_backward(plan, x, w, grad_y, grad_x, grad_w)
    check(lib().fno_spectral_conv3d_backward(plan.handle, _ptr(x), _ptr(w), _ptr(grad_y), _ptr(grad_x),
                                             _ptr(grad_w), _stream(stream, plan.device)),
          "fno_spectral_conv3d_backward")


def fno_plan_saved_bytes(plan):
    """Bytes of the saved-spectra buffer of fno_spectral_conv_forward_save,
    or None when the plan has no saved format (see include/fno.h)."""
    n = ctypes.c_size_t()
    st = lib().fno_plan_saved_bytes(plan.handle, ctypes.byref(n))
    if st == 2:  # FNO_ERR_UNSUPPORTED
        return None
    check(st, "fno_plan_saved_bytes")
    return n.value


def fno_saved_empty(plan):
    """A device buffer (uint8 tensor) for the plan's saved spectra, or None."""
    import torch
    n = fno_plan_saved_bytes(plan)
    if n is None:
        return None
    return torch.empty(n, dtype=torch.uint8, device=f"cuda:{plan.device}")


def _check_saved(plan, saved):
    import torch
    if saved is None or isinstance(saved, int):
        return
    if not isinstance(saved, torch.Tensor):
        raise TypeError("saved must be a torch tensor, a device pointer or None")
    n = fno_plan_saved_bytes(plan)
    if n is None:
        raise ValueError("the plan has no saved-spectra format")
    if saved.numel() * saved.element_size() < n:
        raise ValueError(f"saved holds {saved.numel() * saved.element_size()} bytes, the plan needs {n}")
    if saved.data_ptr() % 256:
        raise ValueError("saved must be 256-byte aligned")


def fno_spectral_conv_forward_save(plan, x, w, y, saved, stream=None):
    """The layer (2D or 3D by the plan) that also leaves the spectra of x in
    `saved` for fno_spectral_conv_backward_saved."""
    _check_tensors(plan, x, w, y)
    _check_saved(plan, saved)
    check(lib().fno_spectral_conv_forward_save(plan.handle, _ptr(x), _ptr(w), _ptr(y), _ptr(saved),
                                               _stream(stream, plan.device)), "fno_spectral_conv_forward_save")


def fno_spectral_conv_backward_saved(plan, saved, w, grad_y, grad_x, grad_w, stream=None):
    """Gradients with the spectra of x read from `saved` (see include/fno.h);
    grad_x or grad_w may be None, saved may be None when grad_w is."""
    _check_backward(plan, None, w, grad_y, grad_x, grad_w)
    _check_saved(plan, saved)
    check(lib().fno_spectral_conv_backward_saved(plan.handle, _ptr(saved), _ptr(w), _ptr(grad_y),
                                                 _ptr(grad_x), _ptr(grad_w), _stream(stream, plan.device)),
          "fno_spectral_conv_backward_saved")


_LAYOUTS = {"split": 0, "corners": 1}


def _check_repack(plan, layout, w, re, im):
    import torch
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}")
    td = _torch_dtype(plan.dtype)
    shape = plan.split_shape() if layout == "split" else plan.corners_shape()
    if layout == "corners" and im is not None:
        raise ValueError("the corner layout is one interleaved array: pass im=None")
    if layout == "split" and im is None:
        raise ValueError("the split layout needs both re and im")
    checks = [("w", w, plan.w_shape()), ("re", re, shape)] + ([("im", im, shape)] if im is not None else [])
    for name, t, want in checks:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.dtype != td:
            raise ValueError(f"{name} dtype {t.dtype} != plan dtype {td}")
        if tuple(t.shape) != tuple(want):
            raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(want)}")


def _as_real(t):
    import torch
    return torch.view_as_real(t) if isinstance(t, torch.Tensor) and t.is_complex() else t


def fno_weights_pack(plan, layout, re, im, w, stream=None):
    """Copy a module's weights into the layer's w. layout "split": re / im of
    plan.split_shape(); "corners": one array of plan.corners_shape() (or the
    complex tensor it is the float view of) and im=None."""
    re = _as_real(re)
    _check_repack(plan, layout, w, re, im)
    check(lib().fno_weights_pack(plan.handle, _LAYOUTS[layout], _ptr(re), _ptr(im), _ptr(w),
                                 _stream(stream, plan.device)), "fno_weights_pack")


def fno_weights_unpack(plan, layout, w, re, im, stream=None):
    """Copy w (or a weight gradient in w's layout) out into a module's layout."""
    re = _as_real(re)
    _check_repack(plan, layout, w, re, im)
    check(lib().fno_weights_unpack(plan.handle, _LAYOUTS[layout], _ptr(w), _ptr(re), _ptr(im),
                                   _stream(stream, plan.device)), "fno_weights_unpack")


def _autograd_function():
    import torch

    class SpectralConvFunction(torch.autograd.Function):
        """The layer as a PyTorch autograd Function on split weights, the
        integration the TurboFNO write-up describes (section 4.3): forward
        takes (input, weight_real, weight_imag), backward returns the three
        gradients. Weight gradients follow PyTorch's convention for a complex
        weight w = weight_real + i weight_imag (dL/dRe, dL/dIm). Every step runs
        in the library's kernels; torch only allocates the tensors."""

        @staticmethod
        def forward(ctx, x, weight_real, weight_imag, plan):
            w = torch.empty(plan.w_shape(), dtype=x.dtype, device=x.device)
            fno_weights_pack(plan, "split", weight_real, weight_imag, w)
            y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
            ctx.plan = plan
            saved = fno_saved_empty(plan)
            if saved is not None:
                # keep the retained spectra of x (what grad_w needs), not x
                fno_spectral_conv_forward_save(plan, x, w, y, saved)
                ctx.save_for_backward(saved, w)
                ctx.kept = "spectra"
            else:
                (fno_spectral_conv2d if plan.ndim == 2 else fno_spectral_conv3d)(plan, x, w, y)
                ctx.save_for_backward(x, w)
                ctx.kept = "x"
            return y

        @staticmethod
        @torch.autograd.function.once_differentiable
        def backward(ctx, grad_y):
            # first derivatives only: a second backward raises instead of
            # silently returning no higher-order terms
            kept, w = ctx.saved_tensors
            plan = ctx.plan
            need_x, need_re, need_im = ctx.needs_input_grad[:3]
            gx = torch.empty(plan.x_shape(), dtype=w.dtype, device=w.device) if need_x else None
            gw = torch.empty_like(w) if (need_re or need_im) else None
            if gx is None and gw is None:
                return None, None, None, None
            if ctx.kept == "spectra":
                fno_spectral_conv_backward_saved(plan, kept if gw is not None else None,
                                                 w if gx is not None else None, grad_y.contiguous(), gx, gw)
            else:
                f = fno_spectral_conv2d_backward if plan.ndim == 2 else fno_spectral_conv3d_backward
                f(plan, kept if gw is not None else None, w if gx is not None else None, grad_y.contiguous(),
                  gx, gw)
            g_re = g_im = None
            if gw is not None:
                g_re = torch.empty(plan.split_shape(), dtype=w.dtype, device=w.device)
                g_im = torch.empty_like(g_re)
                fno_weights_unpack(plan, "split", gw, g_re, g_im)
            return gx, g_re if need_re else None, g_im if need_im else None, None

    return SpectralConvFunction


_FUNCTION = None


def __getattr__(name):
    # the autograd Function subclasses a torch class; build it on first use so
    # importing the binding does not import torch
    global _FUNCTION
    if name == "SpectralConvFunction":
        if _FUNCTION is None:
            _FUNCTION = _autograd_function()
        return _FUNCTION
    raise AttributeError(name)


def spectral_conv(plan, x, weight_real, weight_imag):
    """y = layer(x; weight_real + i weight_imag), differentiable in all three."""
    return __getattr__("SpectralConvFunction").apply(x, weight_real, weight_imag, plan)


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
    """Device pointer of the forward (0) or contracted (1) spectra workspace,
    or (half exchange only) of their exponents (2, 3)."""
    p = ctypes.c_void_p()
    check(lib().fno_plan_spectra(plan.handle, which, ctypes.byref(p)), "fno_plan_spectra")
    return p.value


def fno_plan_spectra_format(plan):
    """0: complex fp32 spectra; 1: fp16 pairs with power-of-two exponents."""
    n = ctypes.c_int()
    check(lib().fno_plan_spectra_format(plan.handle, ctypes.byref(n)), "fno_plan_spectra_format")
    return n.value


LAUNCH_SHAPES = {"separate": 0, "fused": 1, "fused_stall_test": 2}


def fno_plan_set_launch_shape(plan, shape):
    """Launch shape of the plan's forward calls: "separate" (three kernels),
    "fused" (one cooperative launch) or "fused_stall_test" (error-path test)."""
    check(lib().fno_plan_set_launch_shape(plan.handle, LAUNCH_SHAPES[shape]), "fno_plan_set_launch_shape")


def fno_plan_get_launch_shape(plan):
    n = ctypes.c_int()
    check(lib().fno_plan_get_launch_shape(plan.handle, ctypes.byref(n)), "fno_plan_get_launch_shape")
    return {v: k for k, v in LAUNCH_SHAPES.items()}[n.value]


def fno_plan_check(plan):
    """Wait for the device; raises FnoError(FNO_ERR_DEVICE) if a single-launch
    call's barrier wait gave up since the last check."""
    check(lib().fno_plan_check(plan.handle), "fno_plan_check")


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


# ------------------------------------------------------------ FNO2d network

def _dtype_of(t):
    import torch
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def fno_channel_mix(x, A, bias, add, y, act=0, stream=None):
    """y[b][o][p] = act(sum_i A[o][i] x[b][i][p] + bias[o] + add[b][o][p]);
    x [B][Ci][...], y [B][Co][...] (trailing dims flattened to pixels)."""
    B, Ci = x.shape[0], x.shape[1]
    Co = y.shape[1]
    P = x[0, 0].numel()
    dt = _dtype_of(x)
    check(lib().fno_channel_mix(_ptr(x), _ptr(A), _ptr(bias), _ptr(add), _ptr(y), B, Ci, Co, P, act,
                                DTYPES[dt], _stream(stream, x.device.index or 0)), "fno_channel_mix")


def fno_projection(x, Q1, q1, Q2, q2, y, stream=None):
    """y[b][c][p] = sum_j Q2[c][j] GELU(sum_i Q1[j][i] x[b][i][p] + q1[j]) + q2[c]."""
    B, Ci = x.shape[0], x.shape[1]
    J, C = Q1.shape[0], Q2.shape[0]
    P = x[0, 0].numel()
    dt = _dtype_of(x)
    check(lib().fno_projection(_ptr(x), _ptr(Q1), _ptr(q1), _ptr(Q2), _ptr(q2), _ptr(y), B, Ci, J, C, P,
                               DTYPES[dt], _stream(stream, x.device.index or 0)), "fno_projection")


class Model2d:
    """Handle of a C FNO2d model plan plus its shape."""

    def __init__(self, handle, batch, grid, in_channels, channels, n_layers, modes, proj_channels,
                 out_channels, dtype, device):
        self.handle = handle
        self.batch, self.grid, self.in_channels, self.channels = batch, tuple(grid), in_channels, channels
        self.n_layers, self.modes, self.proj_channels = n_layers, tuple(modes), proj_channels
        self.out_channels, self.dtype, self.device = out_channels, dtype, device

    def n_params(self):
        return 2 + 3 * self.n_layers + 4


def fno_model2d_create(batch, grid, in_channels, channels, n_layers, modes, proj_channels, out_channels,
                       dtype="f16", device=0):
    h = ctypes.c_void_p()
    check(lib().fno_model2d_create(ctypes.byref(h), batch, grid[0], grid[1], in_channels, channels, n_layers,
                                   modes[0], modes[1], proj_channels, out_channels, DTYPES[dtype], device),
          "fno_model2d_create")
    return Model2d(h, batch, grid, in_channels, channels, n_layers, modes, proj_channels, out_channels,
                   dtype, device)


def fno_model2d_forward(model, features, params, out, stream=None):
    """params: list of device tensors in the documented order
    [P, p, (spectral w, W, b) * n_layers, Q1, q1, Q2, q2]."""
    if len(params) != model.n_params():
        raise ValueError(f"expected {model.n_params()} parameter tensors, got {len(params)}")
    arr = (ctypes.c_void_p * len(params))(*[_ptr(t) for t in params])
    check(lib().fno_model2d_forward(model.handle, _ptr(features), arr, _ptr(out),
                                    _stream(stream, model.device)), "fno_model2d_forward")


def fno_model2d_set_graph(model, on=True):
    """Replay the model's forward from a captured HIP graph (see include/fno.h)."""
    check(lib().fno_model2d_set_graph(model.handle, 1 if on else 0), "fno_model2d_set_graph")


def fno_model2d_destroy(model):
    if model is None or model.handle is None:
        return
    check(lib().fno_model2d_destroy(model.handle), "fno_model2d_destroy")
    model.handle = None
