"""The single-launch layer (forward planes, contraction and inverse planes in
one cooperative launch joined by grid barriers) through the C ABI: parity with
the float64 oracle in both launch shapes on the same seeded inputs, run-to-run
determinism, one launch per call, and the bounded barrier wait's error report.

The two shapes run the same transforms but split the contraction's input
channels over different numbers of waves, so they agree to rounding, not bit
for bit; each is held to the oracle's tolerance.
"""

import numpy as np
import pytest

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import TOL, rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu


def _cfg(B, Ci, Co, grid, modes, kind="uniform", seed=21):
    return wl.LayerConfig("f", 2, B, Ci, Co, tuple(grid), tuple(modes), ("f32",), seed, kind)


CASES = [
    # VALU planes (register FFTs of 4, 8 and 16 points)
    ("c0", wl.CONFIGS["c0"], "f32"),
    ("valu-mp8-f16", _cfg(3, 5, 3, (32, 64), (5, 3)), "f16"),
    ("valu-mp16-bf16", _cfg(5, 1, 7, (64, 32), (16, 9)), "bf16"),
    ("valu-mp8-sq", _cfg(2, 3, 2, (16, 16), (8, 8)), "f32"),
    # matrix-core planes, W = 64 and 128, partial tiles
    ("mx-c1-b2-f32", _cfg(2, 32, 32, (128, 128), (16, 16), "grf", 1), "f32"),
    ("mx-c1-b2-f16", _cfg(2, 32, 32, (128, 128), (16, 16), "grf", 1), "f16"),
    ("mx-w64-f32", _cfg(3, 2, 2, (64, 64), (5, 8)), "f32"),
    ("mx-w64-bf16", _cfg(3, 5, 2, (128, 64), (13, 5)), "bf16"),
    ("mx-w128-f16", _cfg(1, 3, 6, (64, 128), (16, 16)), "f16"),
    ("mx-ragged-co", _cfg(4, 7, 5, (128, 128), (11, 15)), "f32"),
    # the 128x128 workload at full size
    ("c1-f32", wl.CONFIGS["c1"], "f32"),
    ("c1-f16", wl.CONFIGS["c1"], "f16"),
]


def _run(plan, cfg, dtype, inp, shape):
    import torch
    fno.fno_plan_set_launch_shape(plan, shape)
    x, w = to_device(inp["x"], dtype), to_device(inp["w"], dtype)
    y = torch.full(plan.y_shape(), float("nan"), dtype=x.dtype, device=x.device)
    fno.fno_spectral_conv2d(plan, x, w, y)
    fno.fno_plan_check(plan)
    return to_float64(y)


@pytest.mark.parametrize("name,cfg,dtype", CASES, ids=[c[0] for c in CASES])
def test_fused_parity_both_shapes(name, cfg, dtype):
    print(f"[fused] {name} {dtype}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    ref = oracle.spectral_conv2d(inp["x64"], inp["w64"], *cfg.modes)
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype, 0)
    try:
        assert fno.fno_plan_get_launch_shape(plan) == "separate"
        yf = _run(plan, cfg, dtype, inp, "fused")
        assert fno.fno_plan_num_launches(plan) == 1
        yf2 = _run(plan, cfg, dtype, inp, "fused")
        ys = _run(plan, cfg, dtype, inp, "separate")
        assert fno.fno_plan_num_launches(plan) == 3
    finally:
        fno.fno_plan_destroy(plan)
    assert np.array_equal(yf, yf2), "single launch not deterministic"
    ef, es = rel_l2(yf, ref), rel_l2(ys, ref)
    print(f"[fused] {name}: rel L2 fused {ef:.3e} separate {es:.3e}", flush=True)
    assert ef <= TOL[dtype] and es <= TOL[dtype]


def test_fused_sampled_full_size_grid_reuse():
    # more planes than the co-resident grid: every workgroup loops over
    # several planes and contraction tiles; compared on sampled batch elements
    cfg = wl.LayerConfig("f", 2, 64, 16, 16, (64, 64), (8, 8), ("f32",), 5, "grf")
    inp = wl.layer_inputs(cfg, "f32")
    plan = fno.fno_plan_create(2, 64, 16, 16, (64, 64), (8, 8), "f32", 0)
    try:
        y = _run(plan, cfg, "f32", inp, "fused")
    finally:
        fno.fno_plan_destroy(plan)
    for b in (0, 31, 63):
        ref = oracle.spectral_conv2d(inp["x64"][b:b + 1], inp["w64"], *cfg.modes)
        assert rel_l2(y[b:b + 1], ref) <= TOL["f32"]


def test_stall_test_reports_error_then_recovers():
    import torch
    cfg = wl.CONFIGS["c0"]
    inp = wl.layer_inputs(cfg, "f32")
    ref = oracle.spectral_conv2d(inp["x64"], inp["w64"], *cfg.modes)
    plan = fno.fno_plan_create(2, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, "f32", 0)
    try:
        x, w = to_device(inp["x"], "f32"), to_device(inp["w"], "f32")
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        fno.fno_plan_check(plan)  # nothing pending
        # the barriers wait for one workgroup more than the grid: every wait
        # gives up after its bounded polls and the kernel still finishes
        fno.fno_plan_set_launch_shape(plan, "fused_stall_test")
        fno.fno_spectral_conv2d(plan, x, w, y)
        with pytest.raises(fno.FnoError) as e:
            fno.fno_plan_check(plan)
        assert e.value.status == 4  # FNO_ERR_DEVICE
        fno.fno_plan_check(plan)   # reported once, state reset
        fno.fno_plan_set_launch_shape(plan, "fused")
        fno.fno_spectral_conv2d(plan, x, w, y)
        fno.fno_plan_check(plan)
        assert rel_l2(to_float64(y), ref) <= TOL["f32"]
    finally:
        fno.fno_plan_destroy(plan)


def test_capture_queues_separate_kernels():
    # a captured call of a single-launch plan records the three stand-alone
    # kernels; its replay equals an eager call of those kernels bit for bit
    import torch
    cfg = _cfg(2, 4, 4, (64, 64), (8, 8))
    inp = wl.layer_inputs(cfg, "f32")
    plan = fno.fno_plan_create(2, 2, 4, 4, (64, 64), (8, 8), "f32", 0)
    try:
        x, w = to_device(inp["x"], "f32"), to_device(inp["w"], "f32")
        ref = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        y = torch.empty_like(ref)
        fno.fno_plan_set_launch_shape(plan, "separate")
        fno.fno_spectral_conv2d(plan, x, w, ref)
        fno.fno_plan_set_launch_shape(plan, "fused")
        stream = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fno.fno_spectral_conv2d(plan, x, w, y)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fno.fno_spectral_conv2d(plan, x, w, y)
        for _ in range(2):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ref)
        del g
        fno.fno_plan_check(plan)
    finally:
        torch.cuda.synchronize()
        fno.fno_plan_destroy(plan)
