"""GPU checks of the saved-spectra pair through the C ABI:
fno_spectral_conv_forward_save leaves the retained spectra of x in a caller
buffer and fno_spectral_conv_backward_saved forms the gradients from them
instead of from x. y against the forward oracle and the gradients against
the backward oracle (the bars of the parity tests), and the gradients
against the backward from x on the same plan; a plan without a saved format
says so and keeps working from x; argument errors.

Cases: fp32 matrix-core and register-FFT planes, 3D, fp16 and bf16 layers on
the half exchange (saved fp16 pairs with per-plane exponents), an fp16 layer
exchanging complex fp32; full-size 256x256 fp16 / bf16 against the backward
from x.
"""

import numpy as np
import pytest
import torch

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import TOL, rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu

OK, INVALID, UNSUPPORTED = 0, 1, 2


def _cfg(ndim, B, Ci, Co, grid, modes, kind="grf", seed=31):
    return wl.LayerConfig("s", ndim, B, Ci, Co, tuple(grid), tuple(modes), ("f32",), seed, kind)


def _tensors(plan, cfg, dtype):
    inp = wl.layer_inputs(cfg, dtype)
    gout = wl.layer_grad_output(cfg, dtype)
    x, w, g = to_device(inp["x"], dtype), to_device(inp["w"], dtype), to_device(gout["g"], dtype)
    return inp, gout, x, w, g


def _grads(plan, x, w):
    return (torch.empty(plan.x_shape(), dtype=x.dtype, device=x.device),
            torch.empty(plan.w_shape(), dtype=x.dtype, device=x.device))


def _from_x(plan, x, w, g):
    gx, gw = _grads(plan, x, w)
    f = fno.fno_spectral_conv2d_backward if plan.ndim == 2 else fno.fno_spectral_conv3d_backward
    f(plan, x, w, g, gx, gw)
    torch.cuda.synchronize()
    return to_float64(gx), to_float64(gw)


def _saved_pass(plan, x, w, g):
    y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
    saved = fno.fno_saved_empty(plan)
    assert saved is not None
    fno.fno_spectral_conv_forward_save(plan, x, w, y, saved)
    gx, gw = _grads(plan, x, w)
    fno.fno_spectral_conv_backward_saved(plan, saved, w, g, gx, gw)
    torch.cuda.synchronize()
    return to_float64(y), to_float64(gx), to_float64(gw)


SMALL = [
    ("mx-f32", _cfg(2, 3, 32, 32, (128, 128), (16, 16)), "f32"),
    ("valu-f32", _cfg(2, 3, 5, 3, (32, 64), (5, 3), "uniform"), "f32"),
    ("3d-f32", _cfg(3, 2, 3, 5, (16, 32, 16), (3, 5, 2), "uniform"), "f32"),
    ("hx-f16", _cfg(2, 33, 20, 36, (128, 128), (30, 31), "uniform"), "f16"),
    ("hx-bf16", _cfg(2, 40, 36, 12, (128, 128), (31, 30), "uniform"), "bf16"),
    ("b2-f16", _cfg(2, 2, 32, 24, (128, 128), (16, 16)), "f16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_saved_parity_small(case):
    name, cfg, dtype = case
    print(f"[saved] {name} dtype={dtype} B={cfg.batch} Ci={cfg.c_in} Co={cfg.c_out} grid={cfg.grid} "
          f"modes={cfg.modes}", flush=True)
    plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        inp, gout, x, w, g = _tensors(plan, cfg, dtype)
        y, gx, gw = _saved_pass(plan, x, w, g)
        bx, bw = _from_x(plan, x, w, g)
    finally:
        fno.fno_plan_destroy(plan)
    fwd = oracle.spectral_conv2d if cfg.ndim == 2 else oracle.spectral_conv3d
    bwd = oracle.spectral_conv2d_backward if cfg.ndim == 2 else oracle.spectral_conv3d_backward
    ry = fwd(inp["x64"], inp["w64"], *cfg.modes)
    rx, rw = bwd(inp["x64"], inp["w64"], gout["g64"], *cfg.modes)
    rw = np.stack([rw.real, rw.imag], axis=-1)
    errs = {"y": rel_l2(y, ry), "dx": rel_l2(gx, rx), "dw": rel_l2(gw, rw),
            "dx_vs_from_x": rel_l2(gx, bx), "dw_vs_from_x": rel_l2(gw, bw)}
    print(f"[saved] {name} " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= TOL[dtype], f"{name} {k}: rel L2 {e:.3e}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_saved_full_size(dtype):
    """The 256x256 layer (B=32, 64 -> 64 channels, 32x32 modes) on the half
    exchange: gradients from the saved spectra against those from x."""
    cfg = wl.CONFIGS["c2"]
    print(f"[saved-full] c2 {dtype}", flush=True)
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        n = fno.fno_plan_saved_bytes(plan)
        # fp16 pairs and one int exponent per (b, i) plane
        assert n == cfg.batch * cfg.c_in * cfg.n_modes * 4 + cfg.batch * cfg.c_in * 4
        _, _, x, w, g = _tensors(plan, cfg, dtype)
        _, gx, gw = _saved_pass(plan, x, w, g)
        bx, bw = _from_x(plan, x, w, g)
    finally:
        fno.fno_plan_destroy(plan)
    ex, ew = rel_l2(gx, bx), rel_l2(gw, bw)
    print(f"[saved-full] c2 {dtype} dx_vs_from_x={ex:.3e} dw_vs_from_x={ew:.3e}", flush=True)
    assert ex <= TOL[dtype] and ew <= TOL[dtype]


def test_saved_unsupported_plan():
    """fp16 on the half exchange with K = 2*31*31 (not a multiple of 4): the
    backward keeps complex fp32 spectra, so there is no saved format; the
    gradient of x alone needs none."""
    cfg = _cfg(2, 33, 36, 20, (128, 128), (31, 31), "uniform")
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f16", 0)
    try:
        assert fno.fno_plan_saved_bytes(plan) is None
        inp, gout, x, w, g = _tensors(plan, cfg, "f16")
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        buf = torch.empty(1 << 20, dtype=torch.uint8, device="cuda:0")
        L, p, s = fno.lib(), plan.handle, torch.cuda.current_stream().cuda_stream
        assert L.fno_spectral_conv_forward_save(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), buf.data_ptr(),
                                                s) == UNSUPPORTED
        gx, gw = _grads(plan, x, w)
        assert L.fno_spectral_conv_backward_saved(p, buf.data_ptr(), w.data_ptr(), g.data_ptr(), gx.data_ptr(),
                                                  gw.data_ptr(), s) == INVALID
        fno.fno_spectral_conv_backward_saved(plan, None, w, g, gx, None)
        torch.cuda.synchronize()
        rx, _ = oracle.spectral_conv2d_backward(inp["x64"], inp["w64"], gout["g64"], *cfg.modes)
        assert rel_l2(to_float64(gx), rx) <= TOL["f16"]
    finally:
        fno.fno_plan_destroy(plan)


def test_saved_argument_errors():
    cfg = _cfg(2, 2, 3, 4, (64, 64), (8, 8))
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f32", 0)
    try:
        _, _, x, w, g = _tensors(plan, cfg, "f32")
        y = torch.empty(plan.y_shape(), device="cuda:0")
        n = fno.fno_plan_saved_bytes(plan)
        assert n == ((cfg.batch * cfg.c_in * cfg.n_modes * 8 + 255) // 256) * 256
        buf = torch.empty(n + 512, dtype=torch.uint8, device="cuda:0")
        gx, gw = _grads(plan, x, w)
        L, p, s = fno.lib(), plan.handle, torch.cuda.current_stream().cuda_stream
        sp = buf.data_ptr()
        # NULL or misaligned saved buffer; saved overlapping x or y
        assert L.fno_spectral_conv_forward_save(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), None, s) == INVALID
        assert L.fno_spectral_conv_forward_save(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), sp + 16, s) == INVALID
        assert L.fno_spectral_conv_forward_save(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), y.data_ptr(),
                                                s) == INVALID
        assert L.fno_spectral_conv_forward_save(p, x.data_ptr(), w.data_ptr(), y.data_ptr(), sp, s) == OK
        # grad_w without saved; misaligned saved; an output overlapping saved
        assert L.fno_spectral_conv_backward_saved(p, None, w.data_ptr(), g.data_ptr(), None, gw.data_ptr(),
                                                  s) == INVALID
        assert L.fno_spectral_conv_backward_saved(p, sp + 16, w.data_ptr(), g.data_ptr(), None, gw.data_ptr(),
                                                  s) == INVALID
        assert L.fno_spectral_conv_backward_saved(p, sp, w.data_ptr(), g.data_ptr(), None, sp, s) == INVALID
        assert L.fno_spectral_conv_backward_saved(p, sp, w.data_ptr(), g.data_ptr(), gx.data_ptr(), gw.data_ptr(),
                                                  s) == OK
        torch.cuda.synchronize()
    finally:
        fno.fno_plan_destroy(plan)


def test_saved_forward_ignores_single_launch_shape():
    """A plan set to the single cooperative launch still saves through the
    stand-alone kernels: y and the gradients as from the default shape."""
    cfg = _cfg(2, 3, 32, 32, (128, 128), (16, 16))
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f32", 0)
    try:
        inp, gout, x, w, g = _tensors(plan, cfg, "f32")
        y0, gx0, gw0 = _saved_pass(plan, x, w, g)
        try:
            fno.fno_plan_set_launch_shape(plan, "fused")
        except fno.FnoError:
            pytest.skip("no single-launch shape for this plan on this device")
        y1, gx1, gw1 = _saved_pass(plan, x, w, g)
    finally:
        fno.fno_plan_destroy(plan)
    assert np.array_equal(y0, y1) and np.array_equal(gx0, gx1) and np.array_equal(gw0, gw1)
