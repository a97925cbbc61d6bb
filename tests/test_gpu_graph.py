"""Graph capture of the layer and its backward: a HIP graph captured from one
call (through torch.cuda.graph, on the capture stream the binding picks up)
replays to results bitwise equal to the eager call of the same kernels, every
replay, with eager work and synchronisations between the replays. A plan in
the single-launch shape queues its three stand-alone kernels while the stream
is being captured."""

import numpy as np
import pytest
import torch

import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def _capture(fn):
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("ndim,dtype", [(2, "f32"), (2, "f16"), (3, "f32")])
def test_graph_replay_matches_eager(ndim, dtype):
    if ndim == 2:
        cfg = wl.LayerConfig("g", 2, 4, 8, 12, (128, 128), (16, 16), ("f32",), 31, "grf")
    else:
        cfg = wl.LayerConfig("g", 3, 2, 4, 6, (32, 32, 32), (6, 6, 6), ("f32",), 31, "grf")
    print(f"[graph] ndim={ndim} dtype={dtype}", flush=True)
    plan = fno.fno_plan_create(ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        inp = wl.layer_inputs(cfg, dtype)
        gout = wl.layer_grad_output(cfg, dtype)
        x, w, gy = to_device(inp["x"], dtype), to_device(inp["w"], dtype), to_device(gout["g"], dtype)
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        gx, gw = torch.empty_like(x), torch.empty_like(w)
        fwd = fno.fno_spectral_conv2d if ndim == 2 else fno.fno_spectral_conv3d
        bwd = fno.fno_spectral_conv2d_backward if ndim == 2 else fno.fno_spectral_conv3d_backward
        # under capture a single-launch plan queues its three stand-alone
        # kernels, so the eager reference runs those too
        shape = fno.fno_plan_get_launch_shape(plan)
        fno.fno_plan_set_launch_shape(plan, "separate")
        fwd(plan, x, w, y)
        bwd(plan, x, w, gy, gx, gw)
        torch.cuda.synchronize()
        ref = (y.clone(), gx.clone(), gw.clone())
        fno.fno_plan_set_launch_shape(plan, shape)
        g_fwd = _capture(lambda: fwd(plan, x, w, y))
        g_bwd = _capture(lambda: bwd(plan, x, w, gy, gx, gw))
        for rep in range(3):
            y.zero_()
            gx.zero_()
            gw.zero_()
            torch.cuda.synchronize()
            g_fwd.replay()
            g_bwd.replay()
            torch.cuda.synchronize()
            for name, got, exp in (("y", y, ref[0]), ("grad_x", gx, ref[1]), ("grad_w", gw, ref[2])):
                assert torch.equal(got, exp), f"replay {rep}: {name} differs from the eager call"
            # eager work between replays: another forward on other inputs
            fwd(plan, torch.randn_like(x.float()).to(x.dtype), w, torch.empty_like(y))
            torch.cuda.synchronize()
        del g_fwd, g_bwd
    finally:
        torch.cuda.synchronize()
        fno.fno_plan_destroy(plan)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_graph_training_step_saved_spectra(dtype):
    """The training-step pair (the forward that keeps the spectra of x, then
    the backward from them) captured as one graph replays bitwise equal to
    the eager calls; the fp16 case runs on the half exchange (B = 33,
    20 -> 36 channels, 128x128, modes 30x31), whose saved spectra are fp16
    pairs with per-plane exponents."""
    if dtype == "f32":
        cfg = wl.LayerConfig("g", 2, 4, 8, 12, (128, 128), (16, 16), ("f32",), 31, "grf")
    else:
        cfg = wl.LayerConfig("g", 2, 33, 20, 36, (128, 128), (30, 31), ("f32",), 31, "uniform")
    print(f"[graph-saved] {dtype}", flush=True)
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        inp = wl.layer_inputs(cfg, dtype)
        gout = wl.layer_grad_output(cfg, dtype)
        x, w, gy = to_device(inp["x"], dtype), to_device(inp["w"], dtype), to_device(gout["g"], dtype)
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        gx, gw = torch.empty_like(x), torch.empty_like(w)
        saved = fno.fno_saved_empty(plan)
        assert saved is not None
        saved.zero_()  # the alignment padding between its parts is never written

        def step():
            fno.fno_spectral_conv_forward_save(plan, x, w, y, saved)
            fno.fno_spectral_conv_backward_saved(plan, saved, w, gy, gx, gw)

        step()
        torch.cuda.synchronize()
        ref = (y.clone(), gx.clone(), gw.clone(), saved.clone())
        g = _capture(step)
        for rep in range(3):
            for t in (y, gx, gw, saved):
                t.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for name, got, exp in (("y", y, ref[0]), ("grad_x", gx, ref[1]), ("grad_w", gw, ref[2]),
                                   ("saved", saved, ref[3])):
                assert torch.equal(got, exp), f"replay {rep}: {name} differs from the eager calls"
            # eager work between replays: the plain forward on other inputs
            fno.fno_spectral_conv2d(plan, torch.randn_like(x.float()).to(x.dtype), w, torch.empty_like(y))
            torch.cuda.synchronize()
        del g
    finally:
        torch.cuda.synchronize()
        fno.fno_plan_destroy(plan)
