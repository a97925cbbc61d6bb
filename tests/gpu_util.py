"""Helpers for GPU tests: upload seeded storage arrays, run a layer through the
C ABI, download the result as float64, compare with the oracle."""

import numpy as np

import spectral_convolution_amd as fno

TOL = {"f32": 1e-5, "f16": 3e-3, "bf16": 3e-3}


def to_device(arr, dtype, device="cuda:0"):
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_float64(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    return float(np.linalg.norm((got - ref).ravel()) / np.linalg.norm(ref.ravel()))


def run_layer(ndim, batch, c_in, c_out, grid, modes, dtype, xs, ws, plan=None):
    """Run one layer on cuda:0 from storage arrays; returns (y64, plan)."""
    import torch
    own = plan is None
    if own:
        plan = fno.fno_plan_create(ndim, batch, c_in, c_out, grid, modes, dtype, 0)
    x = to_device(xs, dtype)
    w = to_device(ws, dtype)
    y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
    f = fno.fno_spectral_conv2d if ndim == 2 else fno.fno_spectral_conv3d
    f(plan, x, w, y)
    torch.cuda.synchronize()
    out = to_float64(y)
    if own:
        fno.fno_plan_destroy(plan)
        plan = None
    return out, plan


def read_spectra(plan, which):
    """Copy the plan's spectra workspace (which 0: forward, 1: contracted)."""
    import ctypes
    import torch
    n = plan.batch * (plan.c_in if which == 0 else plan.c_out) * plan.n_modes
    host = np.empty(2 * n, dtype=np.float32)
    torch.cuda.synchronize()
    ptr = fno.fno_plan_spectra(plan, which)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    st = hip.hipMemcpy(host.ctypes.data, ptr, host.nbytes, 2)  # device to host
    assert st == 0, f"hipMemcpy failed: {st}"
    c = host[0::2].astype(np.float64) + 1j * host[1::2].astype(np.float64)
    return c


def _copy_from_device(ptr, host):
    import ctypes
    import torch
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    st = hip.hipMemcpy(host.ctypes.data, ptr, host.nbytes, 2)  # device to host
    assert st == 0, f"hipMemcpy failed: {st}"
    return host


def read_half_spectra(plan, which):
    """Decode the half exchange (fp16 pairs times 2^-exponent) of the forward
    (which 0: one exponent per plane) or contracted (1: one per four modes)
    spectra into complex128 [B][C][K]."""
    C = plan.c_in if which == 0 else plan.c_out
    K = plan.n_modes
    pairs = _copy_from_device(fno.fno_plan_spectra(plan, which), np.empty(plan.batch * C * K * 2, np.float16))
    v = (pairs[0::2].astype(np.float64) + 1j * pairs[1::2].astype(np.float64)).reshape(plan.batch, C, K)
    if which == 0:
        e = _copy_from_device(fno.fno_plan_spectra(plan, 2), np.empty(plan.batch * C, np.int32))
        return v * np.ldexp(1.0, -e.astype(np.int64)).reshape(plan.batch, C, 1)
    kq = (K + 3) // 4
    e = _copy_from_device(fno.fno_plan_spectra(plan, 3), np.empty(plan.batch * C * kq, np.int8))
    e = np.repeat(e.reshape(plan.batch, C, kq).astype(np.int64), 4, axis=2)[:, :, :K]
    return v * np.ldexp(1.0, -e)
