"""GPU parity of the backward pass (grad_x, grad_w) through the C ABI against
the float64 backward oracle on the same seeded inputs. Bar: relative L2 of
each gradient <= 1e-5 for fp32 storage, <= 3e-3 for fp16 / bf16 storage.

* small and ragged shapes (both plane paths, both contraction kernels in the
  adjoint direction, c_in != c_out), compared in full;
* the workload shapes at full size: grad_w in full (it sums over the whole
  batch), grad_x on sampled batch elements (batch elements are independent);
* each output alone (the other NULL), determinism, argument errors.
"""

import numpy as np
import pytest
import torch

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import TOL, rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu


def _cfg(name, ndim, B, Ci, Co, grid, modes, kind="grf", seed=21):
    return wl.LayerConfig(name, ndim, B, Ci, Co, tuple(grid), tuple(modes), ("f32",), seed, kind)


def _backward_gpu(cfg, dtype, inp, gout, want_x=True, want_w=True, plan=None):
    own = plan is None
    if own:
        plan = fno.fno_plan_create(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        x = to_device(inp["x"], dtype)
        w = to_device(inp["w"], dtype)
        g = to_device(gout["g"], dtype)
        gx = torch.empty(plan.x_shape(), dtype=x.dtype, device=x.device) if want_x else None
        gw = torch.empty(plan.w_shape(), dtype=x.dtype, device=x.device) if want_w else None
        f = fno.fno_spectral_conv2d_backward if cfg.ndim == 2 else fno.fno_spectral_conv3d_backward
        f(plan, x, w, g, gx, gw)
        torch.cuda.synchronize()
        rx = to_float64(gx) if want_x else None
        rw = None
        if want_w:
            a = to_float64(gw)
            rw = a[..., 0] + 1j * a[..., 1]
        return rx, rw
    finally:
        if own:
            fno.fno_plan_destroy(plan)


def _oracle(cfg, x64, w64, g64):
    if cfg.ndim == 2:
        return oracle.spectral_conv2d_backward(x64, w64, g64, *cfg.modes)
    return oracle.spectral_conv3d_backward(x64, w64, g64, *cfg.modes)


SMALL = [
    ("c0", wl.CONFIGS["c0"], "f32"),
    ("c1-b3-f32", _cfg("c1s", 2, 3, 32, 32, (128, 128), (16, 16), seed=1), "f32"),
    ("c1-b2-f16", _cfg("c1s", 2, 2, 32, 32, (128, 128), (16, 16), seed=1), "f16"),
    ("c2-b2-f16", _cfg("c2s", 2, 2, 64, 64, (256, 256), (32, 32), seed=2), "f16"),
    ("c2-b2-bf16", _cfg("c2s", 2, 2, 64, 64, (256, 256), (32, 32), seed=2), "bf16"),
    ("c3-b1-f32", _cfg("c3s", 3, 1, 32, 32, (64, 64, 64), (16, 16, 16), seed=3), "f32"),
    # ragged: c_in != c_out both ways, odd sizes, the VALU plane path
    ("rag2d-a", _cfg("r", 2, 3, 5, 3, (32, 64), (5, 3), "uniform"), "f32"),
    ("rag2d-b", _cfg("r", 2, 5, 1, 7, (64, 32), (16, 9), "uniform"), "f16"),
    ("rag2d-m1", _cfg("r", 2, 2, 2, 2, (8, 8), (1, 1), "uniform"), "f32"),
    ("rag2d-wide", _cfg("r", 2, 17, 3, 19, (64, 256), (7, 24), "uniform"), "f32"),
    ("rag3d-a", _cfg("r", 3, 2, 3, 5, (16, 32, 16), (3, 5, 2), "uniform"), "f32"),
    ("rag3d-c", _cfg("r", 3, 3, 2, 1, (32, 16, 64), (16, 8, 5), "uniform"), "bf16"),
    # matrix-core planes and the matrix-core contraction in both directions
    ("mx-2d-rag", _cfg("r", 2, 3, 5, 2, (128, 64), (13, 5), "uniform"), "bf16"),
    ("mx-3d", _cfg("r", 3, 1, 3, 2, (8, 64, 128), (3, 12, 20), "uniform"), "f16"),
    ("cmx-rag-f16", _cfg("r", 2, 33, 20, 36, (128, 128), (30, 31), "uniform"), "f16"),
    ("cmx-rag-bf16", _cfg("r", 2, 40, 36, 12, (128, 128), (31, 30), "uniform"), "bf16"),
    # fp16 forward on the half exchange but K = 2 m1 m2 not a multiple of 4:
    # the backward keeps complex fp32 spectra (the other fp16 matrix-core
    # cases above and the full-size 256x256 one run it on the half exchange)
    ("hx-odd-k-f16", _cfg("r", 2, 33, 36, 20, (128, 128), (31, 31), "uniform"), "f16"),
    ("hx-odd-k-bf16", _cfg("r", 2, 33, 36, 20, (128, 128), (31, 31), "uniform"), "bf16"),
    # 16-row batch tiles in the adjoint contraction (W read transposed)
    ("cmx-b16-f16", _cfg("r", 2, 16, 64, 24, (128, 128), (30, 30), "uniform"), "f16"),
    # the adjoint contraction (64 output channels) on four-mode workgroups,
    # the forward one (24 output channels) below the matrix-core size
    ("cmx-mb4-adjoint-f16", _cfg("r", 2, 20, 64, 24, (128, 128), (24, 24), "uniform"), "f16"),
    # the matrix-core adjoint reads W transposed in 16-byte groups of 4
    # output channels (every matrix-core case above); c_out = 22 keeps the
    # conjugate-transposed copy of W
    ("cmx-wh-f16", _cfg("r", 2, 33, 36, 22, (128, 128), (31, 30), "uniform"), "f16"),
    # weight-gradient tiles: wide batch split over waves, channel tails
    ("gw-split", _cfg("r", 2, 64, 6, 10, (64, 64), (4, 6), "uniform"), "f32"),
    ("gw-ib4", _cfg("r", 2, 4, 48, 40, (64, 64), (20, 28), "uniform"), "f32"),
    # fp32 adjoint contraction reading W directly: the reduction split over
    # two waves with partial step blocks and a partial output tile; over
    # eight waves with partial mode, output and batch tiles. Odd c_out, or
    # an adjoint with 8-row batch tiles, keeps the transposed copy of W
    # (rag2d-a, rag3d-a; adj-wh-bb2).
    ("adj-w-s2", _cfg("r", 2, 8, 64, 26, (64, 64), (32, 32), "uniform"), "f32"),
    ("adj-w-s8", _cfg("r", 2, 3, 20, 34, (64, 64), (5, 7), "uniform"), "f32"),
    ("adj-wh-bb2", _cfg("r", 2, 12, 72, 26, (64, 64), (32, 32), "uniform"), "f32"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_backward_parity_small(case):
    name, cfg, dtype = case
    print(f"[bwd] {name} dtype={dtype} B={cfg.batch} Ci={cfg.c_in} Co={cfg.c_out} grid={cfg.grid} "
          f"modes={cfg.modes}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    gout = wl.layer_grad_output(cfg, dtype)
    gx, gw = _backward_gpu(cfg, dtype, inp, gout)
    rx, rw = _oracle(cfg, inp["x64"], inp["w64"], gout["g64"])
    ex, ew = rel_l2(gx, rx), rel_l2(gw, rw)
    print(f"[bwd] {name} grad_x rel_l2={ex:.3e} grad_w rel_l2={ew:.3e}", flush=True)
    assert ex <= TOL[dtype] and ew <= TOL[dtype], f"{name}: grad_x {ex:.3e} grad_w {ew:.3e}"


@pytest.mark.parametrize("dtype,shift", [("f16", 20), ("bf16", 30)])
def test_backward_half_exchange_wide_batch_range(dtype, shift):
    """Batch elements 1.. of x scaled down by 2^-shift: their spectra planes sit
    2^shift below element 0's, so the weight gradient's per-row rescale takes
    its fp16 product by a subnormal power of two (shift 20) or its fp32 path
    (shift 30, bf16 storage, which holds such inputs). Their contributions
    to grad_w are that much smaller; the result must stay finite and match
    the oracle, dominated by element 0."""
    cfg = _cfg("r", 2, 33, 20, 36, (128, 128), (30, 31), "uniform", seed=7)
    inp = wl.layer_inputs(cfg, dtype)
    x64 = inp["x64"].copy()
    x64[1:] *= 2.0 ** -shift
    xs = wl.generate.round_to_storage(x64, dtype)
    inp = dict(inp, x=xs, x64=wl.generate.storage_to_float64(xs, dtype))
    gout = wl.layer_grad_output(cfg, dtype)
    gx, gw = _backward_gpu(cfg, dtype, inp, gout)
    rx, rw = _oracle(cfg, inp["x64"], inp["w64"], gout["g64"])
    assert np.all(np.isfinite(gw.real)) and np.all(np.isfinite(gw.imag))
    ex, ew = rel_l2(gx, rx), rel_l2(gw, rw)
    print(f"[bwd-range] {dtype} shift={shift} grad_x rel_l2={ex:.3e} grad_w rel_l2={ew:.3e}", flush=True)
    assert ex <= TOL[dtype] and ew <= TOL[dtype]


FULL = [("c1", "f32", (0, 15)), ("c1", "f16", (3,)), ("c2", "f16", (0, 31)), ("c2", "bf16", (17,)),
        ("c3", "f32", (0, 3))]


@pytest.mark.parametrize("case", FULL, ids=[f"{c[0]}-{c[1]}" for c in FULL])
def test_backward_parity_full_size(case):
    name, dtype, samples = case
    cfg = wl.CONFIGS[name]
    print(f"[bwd-full] {name} {dtype} B={cfg.batch} grad_x samples={samples}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    gout = wl.layer_grad_output(cfg, dtype)
    gx, gw = _backward_gpu(cfg, dtype, inp, gout)
    # grad_w sums over the batch: the oracle's full weight gradient
    x64, g64 = inp["x64"], gout["g64"]
    if cfg.ndim == 2:
        gh = oracle.backward.adjoint_inverse2d(g64, *cfg.modes)
        rw = oracle.backward.contract_grad_w(oracle.forward2d(x64, *cfg.modes), gh)
    else:
        gh = oracle.backward.adjoint_inverse3d(g64, *cfg.modes)
        rw = oracle.backward.contract_grad_w(oracle.forward3d(x64, *cfg.modes), gh)
    ew = rel_l2(gw, rw)
    idx = list(samples)
    rx, _ = _oracle(cfg, x64[idx], inp["w64"], g64[idx])
    ex = rel_l2(gx[idx], rx)
    print(f"[bwd-full] {name} {dtype} grad_x rel_l2={ex:.3e} grad_w rel_l2={ew:.3e}", flush=True)
    assert ex <= TOL[dtype] and ew <= TOL[dtype]


@pytest.mark.parametrize("which", ["x", "w"])
def test_backward_single_output(which):
    """Either output alone matches the oracle (the other pointer NULL)."""
    cfg = _cfg("r", 2, 3, 4, 6, (64, 128), (9, 11), "uniform")
    inp = wl.layer_inputs(cfg, "f32")
    gout = wl.layer_grad_output(cfg, "f32")
    gx, gw = _backward_gpu(cfg, "f32", inp, gout, want_x=which == "x", want_w=which == "w")
    rx, rw = _oracle(cfg, inp["x64"], inp["w64"], gout["g64"])
    err = rel_l2(gx, rx) if which == "x" else rel_l2(gw, rw)
    assert err <= TOL["f32"]


def test_backward_deterministic_and_reusable():
    """Two calls on one plan give bitwise-equal gradients, and a forward call
    between them (same workspace) changes nothing."""
    cfg = _cfg("r", 2, 8, 16, 24, (128, 128), (16, 16))
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f16", 0)
    try:
        inp = wl.layer_inputs(cfg, "f16")
        gout = wl.layer_grad_output(cfg, "f16")
        a = _backward_gpu(cfg, "f16", inp, gout, plan=plan)
        x = to_device(inp["x"], "f16")
        w = to_device(inp["w"], "f16")
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        fno.fno_spectral_conv2d(plan, x, w, y)
        b = _backward_gpu(cfg, "f16", inp, gout, plan=plan)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    finally:
        fno.fno_plan_destroy(plan)


def test_backward_argument_errors():
    plan = fno.fno_plan_create(2, 2, 3, 4, (64, 64), (8, 8), "f32", 0)
    plan3 = fno.fno_plan_create(3, 1, 2, 2, (16, 16, 16), (4, 4, 4), "f32", 0)
    try:
        x = torch.zeros(plan.x_shape(), device="cuda:0")
        w = torch.zeros(plan.w_shape(), device="cuda:0")
        g = torch.zeros(plan.y_shape(), device="cuda:0")
        gx = torch.empty_like(x)
        gw = torch.empty_like(w)
        L = fno.lib()
        s = torch.cuda.current_stream().cuda_stream
        INVALID = 1
        p = plan.handle
        # both outputs NULL; grad_y NULL; an input an output needs is NULL
        assert L.fno_spectral_conv2d_backward(p, x.data_ptr(), w.data_ptr(), g.data_ptr(), None, None, s) == INVALID
        assert L.fno_spectral_conv2d_backward(p, x.data_ptr(), w.data_ptr(), None, gx.data_ptr(), None, s) == INVALID
        assert L.fno_spectral_conv2d_backward(p, None, w.data_ptr(), g.data_ptr(), None, gw.data_ptr(), s) == INVALID
        assert L.fno_spectral_conv2d_backward(p, x.data_ptr(), None, g.data_ptr(), gx.data_ptr(), None, s) == INVALID
        # misaligned output, output overlapping an input, wrong ndim
        assert L.fno_spectral_conv2d_backward(p, x.data_ptr(), w.data_ptr(), g.data_ptr(), gx.data_ptr() + 4, None,
                                              s) == INVALID
        assert L.fno_spectral_conv2d_backward(p, x.data_ptr(), w.data_ptr(), g.data_ptr(), g.data_ptr(), None,
                                              s) == INVALID
        assert L.fno_spectral_conv3d_backward(p, x.data_ptr(), w.data_ptr(), g.data_ptr(), gx.data_ptr(), None,
                                              s) == INVALID
        assert L.fno_spectral_conv2d_backward(plan3.handle, x.data_ptr(), w.data_ptr(), g.data_ptr(), gx.data_ptr(),
                                              None, s) == INVALID
        # the valid call still works after the rejected ones
        fno.fno_spectral_conv2d_backward(plan, x, w, g, gx, gw)
        torch.cuda.synchronize()
        assert float(gx.abs().max()) == 0.0 and float(gw.abs().max()) == 0.0
    finally:
        fno.fno_plan_destroy(plan)
        fno.fno_plan_destroy(plan3)
