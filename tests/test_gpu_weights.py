"""Weight layouts and the autograd Function, on the GPU through the C ABI.

* fno_weights_pack / fno_weights_unpack move elements only, so they are
  compared bit for bit with layouts built here on the host by numpy
  reshapes and transposes of the workload's own w.
* The corner layout's meaning (which weights act on which spectrum corner)
  is pinned by the layer's output against the common FNO module's
  definition written with numpy.fft: rfft2 / rfftn, per-corner einsum over
  the input channel on the sliced spectrum, irfft2 / irfftn.
* spectral_conv (the autograd Function on split weights) against the
  float64 backward oracle: y, dL/dx, dL/dRe w, dL/dIm w.
"""

import numpy as np
import pytest
import torch

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import TOL, rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu


def _cfg(ndim, B, Ci, Co, grid, modes, seed=31):
    return wl.LayerConfig("wt", ndim, B, Ci, Co, tuple(grid), tuple(modes), ("f32",), seed, "uniform")


def _bits(t):
    a = t.cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return a.numpy().view(np.uint16 if a.element_size() == 2 else np.uint32)


def _host_bits(arr):
    return np.ascontiguousarray(arr).view(np.uint16 if arr.itemsize == 2 else np.uint32)


def _corners_from_w(w, ndim, Ci, Co, modes):
    """Stacked per-corner, channels-first layout of w ([modes][Ci][Co][2])."""
    if ndim == 2:
        m1, m2 = modes
        a = w.reshape(2, m1, m2, Ci, Co, 2)              # corner, kx', ky, i, o, re/im
        return np.ascontiguousarray(a.transpose(0, 3, 4, 1, 2, 5))
    m1, m2, m3 = modes
    a = w.reshape(2, m1, 2, m2, m3, Ci, Co, 2)           # cx, kx', cy, ky', kz, i, o, re/im
    a = a.transpose(2, 0, 5, 6, 1, 3, 4, 7)              # corner index cx + 2 cy: cy outer
    return np.ascontiguousarray(a.reshape(4, Ci, Co, m1, m2, m3, 2))


CASES = [(_cfg(2, 1, 3, 5, (32, 64), (5, 7)), "f32"), (_cfg(2, 1, 4, 2, (64, 64), (8, 3)), "f16"),
         (_cfg(2, 1, 2, 3, (16, 16), (4, 8)), "bf16"), (_cfg(3, 1, 3, 2, (16, 16, 16), (3, 2, 5)), "f32"),
         (_cfg(3, 1, 2, 2, (8, 16, 8), (4, 1, 2)), "bf16")]
IDS = [f"{c.ndim}d-{d}-{c.c_in}x{c.c_out}-m{'x'.join(map(str, c.modes))}" for c, d in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_pack_unpack_bitwise(case):
    cfg, dtype = case
    print(f"[weights] {cfg.ndim}d {dtype} modes={cfg.modes}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    w_host = inp["w"]
    plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        want = _host_bits(w_host)
        # split: the modes-first real and imaginary arrays
        re = to_device(np.ascontiguousarray(w_host[..., 0]), dtype)
        im = to_device(np.ascontiguousarray(w_host[..., 1]), dtype)
        w = torch.full(plan.w_shape(), 7.0, dtype=re.dtype, device=re.device)
        fno.fno_weights_pack(plan, "split", re, im, w)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(w), want)
        re2, im2 = torch.zeros_like(re), torch.zeros_like(im)
        fno.fno_weights_unpack(plan, "split", w, re2, im2)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(re2), _bits(re)) and np.array_equal(_bits(im2), _bits(im))
        # corners: stacked per-corner, channels first
        corners = _corners_from_w(w_host, cfg.ndim, cfg.c_in, cfg.c_out, cfg.modes)
        assert corners.shape == plan.corners_shape()
        cd = to_device(corners, dtype)
        w2 = torch.full(plan.w_shape(), 7.0, dtype=re.dtype, device=re.device)
        fno.fno_weights_pack(plan, "corners", cd, None, w2)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(w2), want)
        back = torch.zeros_like(cd)
        fno.fno_weights_unpack(plan, "corners", w2, back, None)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(back), _host_bits(corners))
    finally:
        fno.fno_plan_destroy(plan)


def _module_definition(x, corners, ndim, modes):
    """The common FNO module's layer in float64 with numpy.fft: one complex
    weight per spectrum corner, channels first."""
    if ndim == 2:
        m1, m2 = modes
        H, W = x.shape[2:]
        xf = np.fft.rfft2(x)
        out = np.zeros((x.shape[0], corners.shape[2], H, W // 2 + 1), complex)
        out[:, :, :m1, :m2] = np.einsum("bixy,ioxy->boxy", xf[:, :, :m1, :m2], corners[0])
        out[:, :, H - m1:, :m2] = np.einsum("bixy,ioxy->boxy", xf[:, :, H - m1:, :m2], corners[1])
        return np.fft.irfft2(out, s=(H, W))
    m1, m2, m3 = modes
    X, Y, Z = x.shape[2:]
    xf = np.fft.rfftn(x, axes=(2, 3, 4))
    out = np.zeros((x.shape[0], corners.shape[2], X, Y, Z // 2 + 1), complex)
    sx = [slice(0, m1), slice(X - m1, X)]
    sy = [slice(0, m2), slice(Y - m2, Y)]
    for cy in range(2):
        for cx in range(2):
            s = (slice(None), slice(None), sx[cx], sy[cy], slice(0, m3))
            out[s] = np.einsum("bixyz,ioxyz->boxyz", xf[s], corners[cx + 2 * cy])
    return np.fft.irfftn(out, s=(X, Y, Z), axes=(2, 3, 4))


@pytest.mark.parametrize("ndim", [2, 3])
def test_corner_layout_meaning(ndim):
    cfg = _cfg(2, 2, 3, 4, (32, 16), (6, 5)) if ndim == 2 else _cfg(3, 2, 2, 3, (16, 16, 16), (4, 3, 5))
    print(f"[weights-corners] {ndim}d grid={cfg.grid} modes={cfg.modes}", flush=True)
    rng = np.random.default_rng(5)
    x64 = rng.standard_normal((cfg.batch, cfg.c_in) + cfg.grid)
    ncorner = 2 if ndim == 2 else 4
    c64 = rng.uniform(-1, 1, (ncorner, cfg.c_in, cfg.c_out) + cfg.modes + (2,))
    xs, cs = x64.astype(np.float32), c64.astype(np.float32)
    plan = fno.fno_plan_create(ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f32", 0)
    try:
        x, cd = to_device(xs, "f32"), to_device(cs, "f32")
        w = torch.empty(plan.w_shape(), dtype=torch.float32, device="cuda:0")
        fno.fno_weights_pack(plan, "corners", torch.view_as_complex(cd), None, w)
        y = torch.empty(plan.y_shape(), dtype=torch.float32, device="cuda:0")
        (fno.fno_spectral_conv2d if ndim == 2 else fno.fno_spectral_conv3d)(plan, x, w, y)
        torch.cuda.synchronize()
        got = to_float64(y)
    finally:
        fno.fno_plan_destroy(plan)
    cplx = cs.astype(np.float64)[..., 0] + 1j * cs.astype(np.float64)[..., 1]
    ref = _module_definition(xs.astype(np.float64), cplx, ndim, cfg.modes)
    err = rel_l2(got, ref)
    print(f"[weights-corners] {ndim}d rel_l2={err:.3e}", flush=True)
    assert err <= 1e-5


# the Function keeps the saved spectra of x where the plan has a saved
# format (every case but the last), else x: the fp16 layer on the half
# exchange with K = 2*31*31 has none
AG = [(_cfg(2, 3, 4, 5, (64, 64), (8, 12)), "f32"), (_cfg(2, 2, 6, 4, (128, 64), (16, 9)), "f16"),
      (_cfg(3, 2, 3, 2, (16, 16, 8), (4, 3, 2)), "f32"),
      (_cfg(2, 33, 20, 36, (128, 128), (30, 31)), "f16"), (_cfg(2, 40, 36, 12, (128, 128), (31, 30)), "bf16"),
      (_cfg(2, 33, 36, 20, (128, 128), (31, 31)), "f16")]


@pytest.mark.parametrize("case", AG, ids=[f"{c.ndim}d-{d}-b{c.batch}-k{c.n_modes}" for c, d in AG])
def test_autograd_function(case):
    cfg, dtype = case
    print(f"[autograd] {cfg.ndim}d {dtype} grid={cfg.grid}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    gout = wl.layer_grad_output(cfg, dtype)
    plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        x = to_device(inp["x"], dtype).requires_grad_(True)
        re = to_device(np.ascontiguousarray(inp["w"][..., 0]), dtype).requires_grad_(True)
        im = to_device(np.ascontiguousarray(inp["w"][..., 1]), dtype).requires_grad_(True)
        g = to_device(gout["g"], dtype)
        y = fno.spectral_conv(plan, x, re, im)
        y.backward(g)
        torch.cuda.synchronize()
        dx_ref, dw_ref = (oracle.spectral_conv2d_backward if cfg.ndim == 2 else oracle.spectral_conv3d_backward)(
            inp["x64"], inp["w64"], gout["g64"], *cfg.modes)
        y_ref = (oracle.spectral_conv2d if cfg.ndim == 2 else oracle.spectral_conv3d)(
            inp["x64"], inp["w64"], *cfg.modes)
        errs = {"y": rel_l2(to_float64(y.detach()), y_ref), "dx": rel_l2(to_float64(x.grad), dx_ref),
                "dw": rel_l2(to_float64(re.grad) + 1j * to_float64(im.grad), dw_ref)}
        print(f"[autograd] {errs}", flush=True)
        for k, e in errs.items():
            assert e <= TOL[dtype], f"{k}: rel L2 {e:.3e}"
        # only the weights need a gradient: dL/dx is skipped
        x2 = x.detach()
        re.grad = im.grad = None
        fno.spectral_conv(plan, x2, re, im).backward(g)
        torch.cuda.synchronize()
        assert rel_l2(to_float64(re.grad) + 1j * to_float64(im.grad), dw_ref) <= TOL[dtype]
        # first derivatives only: differentiating the backward raises
        (gx,) = torch.autograd.grad(fno.spectral_conv(plan, x, re, im), x, g, create_graph=True)
        with pytest.raises(RuntimeError):
            gx.sum().backward()
        torch.cuda.synchronize()
    finally:
        fno.fno_plan_destroy(plan)


def test_repack_argument_errors():
    plan = fno.fno_plan_create(2, 1, 2, 3, (16, 16), (4, 4), "f32", 0)
    try:
        w = torch.empty(plan.w_shape(), device="cuda:0")
        re = torch.empty(plan.split_shape(), device="cuda:0")
        with pytest.raises(ValueError):
            fno.fno_weights_pack(plan, "split", re, None, w)
        with pytest.raises(ValueError):
            fno.fno_weights_pack(plan, "corners", re, re, w)
        with pytest.raises(ValueError):
            fno.fno_weights_pack(plan, "rows", re, re, w)
        with pytest.raises(ValueError):
            fno.fno_weights_pack(plan, "split", re.half(), re.half(), w)
        lib = fno.lib()
        p = w.data_ptr()
        assert lib.fno_weights_pack(plan.handle, 0, re.data_ptr(), None, p, None) == 1   # im missing
        assert lib.fno_weights_pack(plan.handle, 1, re.data_ptr(), re.data_ptr(), p, None) == 1
        assert lib.fno_weights_pack(plan.handle, 2, re.data_ptr(), re.data_ptr(), p, None) == 1
        assert lib.fno_weights_pack(plan.handle, 0, p, p + 8, p, None) == 1   # w overlaps re
        assert lib.fno_weights_pack(plan.handle, 0, re.data_ptr() + 2, p, p, None) == 1  # misaligned
    finally:
        fno.fno_plan_destroy(plan)
