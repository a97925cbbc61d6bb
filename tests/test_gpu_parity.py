"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs. Bar: relative L2 over the compared output <= 1e-5 for
fp32 storage, <= 3e-3 for fp16 / bf16 storage.

* small and ragged shapes, compared element by element in full;
* the five workload shapes at full size in the launch configuration the
  benchmark times, compared on sampled batch elements (the oracle runs on
  those samples only; batch elements are independent);
* the intermediate spectra, determinism, launch structure and error paths.
"""

import ctypes

import numpy as np
import pytest

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import TOL, read_half_spectra, read_spectra, rel_l2, run_layer, to_device

pytestmark = pytest.mark.gpu


def _cfg(name, ndim, B, Ci, Co, grid, modes, kind="grf", seed=11):
    return wl.LayerConfig(name, ndim, B, Ci, Co, tuple(grid), tuple(modes), ("f32",), seed, kind)


def _oracle(cfg, x64, w64):
    if cfg.ndim == 2:
        return oracle.spectral_conv2d(x64, w64, *cfg.modes)
    return oracle.spectral_conv3d(x64, w64, *cfg.modes)


SMALL = [
    ("c0", wl.CONFIGS["c0"], "f32"),
    ("c1-b2-f32", _cfg("c1s", 2, 2, 32, 32, (128, 128), (16, 16), seed=1), "f32"),
    ("c1-b2-f16", _cfg("c1s", 2, 2, 32, 32, (128, 128), (16, 16), seed=1), "f16"),
    ("c2-b1-f16", _cfg("c2s", 2, 1, 64, 64, (256, 256), (32, 32), seed=2), "f16"),
    ("c2-b1-bf16", _cfg("c2s", 2, 1, 64, 64, (256, 256), (32, 32), seed=2), "bf16"),
    ("c3-b1-f32", _cfg("c3s", 3, 1, 32, 32, (64, 64, 64), (16, 16, 16), seed=3), "f32"),
    # ragged: odd channel counts and batch, non-square grids, modes that are
    # not powers of two, the smallest and the largest register FFT
    ("rag2d-a", _cfg("r", 2, 3, 5, 3, (32, 64), (5, 3), "uniform"), "f32"),
    ("rag2d-b", _cfg("r", 2, 5, 1, 7, (64, 32), (16, 9), "uniform"), "f16"),
    ("rag2d-m1", _cfg("r", 2, 2, 2, 2, (8, 8), (1, 1), "uniform"), "f32"),
    ("rag2d-max", _cfg("r", 2, 2, 3, 2, (16, 16), (8, 8), "uniform"), "f32"),
    ("rag2d-tall", _cfg("r", 2, 2, 4, 6, (256, 64), (3, 32), "uniform"), "bf16"),
    ("rag2d-wide", _cfg("r", 2, 17, 3, 19, (64, 256), (7, 24), "uniform"), "f32"),
    ("rag2d-mp2", _cfg("r", 2, 1, 2, 3, (256, 256), (1, 2), "uniform"), "f32"),
    ("rag3d-a", _cfg("r", 3, 2, 3, 5, (16, 32, 16), (3, 5, 2), "uniform"), "f32"),
    ("rag3d-b", _cfg("r", 3, 1, 4, 4, (8, 8, 8), (4, 4, 4), "uniform"), "f16"),
    ("rag3d-c", _cfg("r", 3, 3, 2, 1, (32, 16, 64), (16, 8, 5), "uniform"), "bf16"),
    # fp16 / bf16 planes on the matrix-core path: partial tiles in every
    # product, the largest and smallest mode counts, 3D slabs
    ("mx-2d-rag", _cfg("r", 2, 3, 5, 2, (128, 64), (13, 5), "uniform"), "bf16"),
    ("mx-2d-m1max", _cfg("r", 2, 1, 2, 3, (64, 256), (32, 32), "uniform"), "f16"),
    ("mx-2d-m1", _cfg("r", 2, 2, 3, 1, (64, 64), (1, 1), "uniform"), "bf16"),
    ("mx-2d-c4", _cfg("r", 2, 1, 4, 4, (256, 256), (24, 24)), "f16"),
    ("mx-3d", _cfg("r", 3, 1, 3, 2, (8, 64, 128), (3, 12, 20), "uniform"), "f16"),
    # forward workgroup shapes: 8 waves for more than four m-tiles with one
    # or two R c-tiles per wave, 4 waves with one, split fp32 operands on
    # every shape they take
    ("mx-nw8-cpw1", _cfg("r", 2, 2, 3, 2, (64, 64), (20, 12), "uniform"), "f16"),
    ("mx-nw8-cpw2", _cfg("r", 2, 1, 2, 3, (128, 128), (24, 20), "uniform"), "bf16"),
    ("mx-w256-cpw1", _cfg("r", 2, 1, 3, 2, (64, 256), (9, 14), "uniform"), "f16"),
    ("mx-f32-nt4", _cfg("r", 2, 2, 2, 3, (64, 128), (10, 24), "uniform"), "f32"),
    ("mx-f32-nw8", _cfg("r", 2, 1, 3, 2, (128, 64), (18, 7), "uniform"), "f32"),
    ("mx-f32-nt1", _cfg("r", 2, 3, 2, 2, (64, 64), (5, 8), "uniform"), "f32"),
    ("mx-f32-m2", _cfg("r", 2, 2, 2, 3, (64, 64), (20, 20), "uniform"), "f32"),
    # fp16 / bf16 contraction on matrix cores: ragged batch, channel and mode
    # tiles (two batch tiles, partial input stages, partial output tiles)
    ("cmx-rag-f16", _cfg("r", 2, 33, 20, 36, (128, 128), (30, 31), "uniform"), "f16"),
    ("cmx-rag-bf16", _cfg("r", 2, 40, 33, 12, (128, 128), (31, 30), "uniform"), "bf16"),
    # four-mode workgroups (fewer than two eight-mode workgroups per CU):
    # one and two batch tiles, fp16 and bf16 weights
    ("cmx-mb4-f16", _cfg("r", 2, 16, 64, 64, (128, 128), (24, 24), "uniform"), "f16"),
    ("cmx-mb4-f16-b20", _cfg("r", 2, 20, 24, 64, (128, 128), (24, 24), "uniform"), "f16"),
    ("cmx-mb4-bf16-b20", _cfg("r", 2, 20, 40, 64, (64, 128), (28, 21), "uniform"), "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_parity_small(case):
    name, cfg, dtype = case
    print(f"[parity] {name} dtype={dtype} grid={cfg.grid} modes={cfg.modes}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    got, _ = run_layer(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype,
                       inp["x"], inp["w"])
    ref = _oracle(cfg, inp["x64"], inp["w64"])
    err = rel_l2(got, ref)
    print(f"[parity] {name} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype], f"{name}: rel L2 {err:.3e} > {TOL[dtype]}"


@pytest.mark.parametrize("dtype,scale", [("f16", 2.0 ** -12), ("f16", 2.0 ** 10), ("bf16", 2.0 ** -60),
                                         ("bf16", 2.0 ** 60)])
def test_parity_magnitude(dtype, scale):
    """The half-precision plane products rescale by powers of two chosen from
    the data; inputs far from unit magnitude must keep the same accuracy."""
    cfg = _cfg("m", 2, 2, 3, 4, (128, 128), (16, 16), seed=7)
    inp = wl.layer_inputs(cfg, dtype)
    xs = wl.round_to_storage(inp["x64"] * scale, dtype)
    x64 = wl.storage_to_float64(xs, dtype)
    got, _ = run_layer(2, 2, 3, 4, cfg.grid, cfg.modes, dtype, xs, inp["w"])
    ref = oracle.spectral_conv2d(x64, inp["w64"], *cfg.modes)
    err = rel_l2(got, ref)
    print(f"[parity-mag] {dtype} scale={scale:.3g} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype]


# the 128x128 layer is compared on every batch element, the others on samples
FULL = [("c1", "f32", tuple(range(16))), ("c1", "f16", tuple(range(16))), ("c2", "f16", (0, 31)),
        ("c2", "bf16", (0, 31)), ("c3", "f32", (0, 3))]


@pytest.mark.parametrize("case", FULL, ids=[f"{c[0]}-{c[1]}" for c in FULL])
def test_parity_full_size_sampled(case):
    name, dtype, samples = case
    cfg = wl.CONFIGS[name]
    print(f"[parity-full] {name} {dtype} B={cfg.batch} samples={len(samples)}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    got, _ = run_layer(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype,
                       inp["x"], inp["w"])
    idx = list(samples)
    ref = _oracle(cfg, inp["x64"][idx], inp["w64"])
    err = rel_l2(got[idx], ref)
    print(f"[parity-full] {name} {dtype} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype]
    assert np.isfinite(got).all()


# many planes per persistent workgroup: the forward's register ring and the
# inverse's spectra prefetch cross plane boundaries many times
MANY = [("many-f16-64", _cfg("r", 2, 8, 96, 80, (64, 64), (20, 11), "uniform"), "f16", (0, 7)),
        ("many-bf16-128", _cfg("r", 2, 4, 70, 90, (128, 128), (9, 24), "uniform"), "bf16", (1, 3)),
        ("many-f32-64x128", _cfg("r", 2, 6, 64, 64, (64, 128), (16, 16), "uniform"), "f32", (0, 5))]


@pytest.mark.parametrize("case", MANY, ids=[c[0] for c in MANY])
def test_parity_many_planes(case):
    name, cfg, dtype, samples = case
    print(f"[parity-many] {name} dtype={dtype} B={cfg.batch} Ci={cfg.c_in} Co={cfg.c_out}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    got, _ = run_layer(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype,
                       inp["x"], inp["w"])
    idx = list(samples)
    ref = _oracle(cfg, inp["x64"][idx], inp["w64"])
    err = rel_l2(got[idx], ref)
    print(f"[parity-many] {name} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype]
    assert np.isfinite(got).all()


# The largest axis (256) and the largest retained-mode count (32 per axis)
# on every kernel family: the VALU plane path at its widest register FFT
# (fp32, 256 wide), the 3D x-axis pass over 256 slabs, the matrix-core plane
# path inside a 3D plan at 256 x 256, and a 256-long x axis with 32 kx.
MAXIMA = [
    ("max2d-valu-f32", _cfg("x", 2, 1, 2, 1, (256, 256), (32, 32), "uniform"), "f32"),
    ("max3d-axis-f32", _cfg("x", 3, 1, 1, 2, (256, 64, 256), (32, 16, 32), "uniform"), "f32"),
    ("max3d-mx-f16", _cfg("x", 3, 1, 2, 1, (64, 256, 256), (32, 32, 32), "uniform"), "f16"),
    ("max3d-mx-bf16", _cfg("x", 3, 1, 1, 1, (256, 128, 128), (32, 32, 32), "uniform"), "bf16"),
]


@pytest.mark.parametrize("case", MAXIMA, ids=[c[0] for c in MAXIMA])
def test_parity_maximum_sizes(case):
    name, cfg, dtype = case
    print(f"[parity-max] {name} grid={cfg.grid} modes={cfg.modes}", flush=True)
    inp = wl.layer_inputs(cfg, dtype)
    got, _ = run_layer(cfg.ndim, cfg.batch, cfg.c_in, cfg.c_out, cfg.grid, cfg.modes, dtype,
                       inp["x"], inp["w"])
    err = rel_l2(got, _oracle(cfg, inp["x64"], inp["w64"]))
    print(f"[parity-max] {name} rel_l2={err:.3e}", flush=True)
    assert err <= TOL[dtype]


# Several plans alive at once that share kernel instantiations but need
# different amounts of LDS: each kernel's LDS allowance is per kernel, not per
# plan, so preparing a smaller plan after a larger one must not shrink it.
LIVE = [
    ("live-f32", [_cfg("a", 2, 2, 3, 2, (64, 256), (20, 24), "uniform"),
                  _cfg("b", 2, 1, 2, 3, (64, 64), (5, 8), "uniform")], "f32"),
    ("live-f16", [_cfg("a", 2, 1, 4, 4, (256, 256), (24, 24), "uniform"),
                  _cfg("b", 2, 33, 20, 36, (128, 128), (30, 31), "uniform"),
                  _cfg("c", 2, 2, 3, 1, (64, 64), (1, 1), "uniform")], "f16"),
    ("live-3d", [_cfg("a", 3, 1, 4, 4, (32, 64, 64), (8, 16, 16), "uniform"),
                 _cfg("b", 3, 1, 2, 2, (8, 8, 8), (2, 2, 2), "uniform")], "f32"),
]


@pytest.mark.parametrize("case", LIVE, ids=[c[0] for c in LIVE])
def test_parity_live_plans(case):
    name, cfgs, dtype = case
    plans = [fno.fno_plan_create(c.ndim, c.batch, c.c_in, c.c_out, c.grid, c.modes, dtype, 0)
             for c in cfgs]
    try:
        # run in creation order: every plan after the first was prepared later
        for c, plan in zip(cfgs, plans):
            print(f"[parity-live] {name} grid={c.grid} modes={c.modes} B={c.batch}", flush=True)
            inp = wl.layer_inputs(c, dtype)
            got, _ = run_layer(c.ndim, c.batch, c.c_in, c.c_out, c.grid, c.modes, dtype,
                               inp["x"], inp["w"], plan=plan)
            err = rel_l2(got, _oracle(c, inp["x64"], inp["w64"]))
            print(f"[parity-live] {name} rel_l2={err:.3e}", flush=True)
            assert err <= TOL[dtype]
    finally:
        for plan in plans:
            fno.fno_plan_destroy(plan)


def test_intermediate_spectra():
    cfg = _cfg("s", 2, 2, 3, 4, (64, 128), (6, 11), "uniform")
    inp = wl.layer_inputs(cfg, "f32")
    _, plan = run_layer(2, 2, 3, 4, cfg.grid, cfg.modes, "f32", inp["x"], inp["w"],
                        plan=fno.fno_plan_create(2, 2, 3, 4, cfg.grid, cfg.modes, "f32", 0))
    try:
        xh = read_spectra(plan, 0).reshape(2, 3, 12, 11)
        ref = oracle.forward2d(inp["x64"], *cfg.modes) / (64 * 128)
        assert rel_l2(xh, ref) <= 1e-6
        yh = read_spectra(plan, 1).reshape(2, 4, 12, 11)
        ref_y = oracle.contract(ref, inp["w64"])
        assert rel_l2(yh, ref_y) <= 1e-6
    finally:
        fno.fno_plan_destroy(plan)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_intermediate_half_spectra(dtype):
    # fp16 / bf16 plans on the matrix-core planes and contraction exchange
    # the spectra as fp16 pairs with power-of-two exponents; decoded, they
    # match the oracle's spectra of the same storage-rounded inputs to the
    # fp16 rounding (2^-11 relative) plus the transforms' own error
    cfg = _cfg("s", 2, 16, 8, 32, (64, 64), (32, 32), "grf", seed=7)
    inp = wl.layer_inputs(cfg, dtype)
    plan = fno.fno_plan_create(2, 16, 8, 32, cfg.grid, cfg.modes, dtype, 0)
    try:
        assert fno.fno_plan_spectra_format(plan) == 1
        y, _ = run_layer(2, 16, 8, 32, cfg.grid, cfg.modes, dtype, inp["x"], inp["w"], plan=plan)
        xh = read_half_spectra(plan, 0).reshape(16, 8, 64, 32)
        ref = oracle.forward2d(inp["x64"], *cfg.modes) / (64 * 64)
        ex = rel_l2(xh, ref)
        yh = read_half_spectra(plan, 1).reshape(16, 32, 64, 32)
        ey = rel_l2(yh, oracle.contract(ref, inp["w64"]))
        ez = rel_l2(y, oracle.spectral_conv2d(inp["x64"], inp["w64"], *cfg.modes))
        print(f"[half-spectra] {dtype}: forward {ex:.2e} contracted {ey:.2e} output {ez:.2e}", flush=True)
        assert ex <= 1e-3 and ey <= 1.5e-3 and ez <= TOL[dtype]
    finally:
        fno.fno_plan_destroy(plan)


def test_half_spectra_tiny_and_large_inputs():
    # the exponents follow the data: inputs 2^-40 and 2^+10 times the
    # workload's (bf16 storage, far outside fp16's range either way) give the
    # same relative error as unit-scale inputs
    cfg = _cfg("s", 2, 16, 4, 32, (64, 64), (32, 32), "grf", seed=8)
    inp = wl.layer_inputs(cfg, "bf16")
    plan = fno.fno_plan_create(2, 16, 4, 32, cfg.grid, cfg.modes, "bf16", 0)
    try:
        errs = []
        for sc in (2.0 ** -40, 1.0, 2.0 ** 10):
            xs = wl.round_to_storage(inp["x64"] * sc, "bf16")
            x64 = wl.storage_to_float64(xs, "bf16")
            y, _ = run_layer(2, 16, 4, 32, cfg.grid, cfg.modes, "bf16", xs, inp["w"], plan=plan)
            errs.append(rel_l2(y, oracle.spectral_conv2d(x64, inp["w64"], *cfg.modes)))
        print(f"[half-spectra] scales 2^-40, 1, 2^10: {errs}", flush=True)
        assert max(errs) <= TOL["bf16"]
    finally:
        fno.fno_plan_destroy(plan)


def test_intermediate_spectra_3d():
    cfg = _cfg("s", 3, 1, 2, 3, (16, 32, 16), (4, 6, 3), "uniform")
    inp = wl.layer_inputs(cfg, "f32")
    plan = fno.fno_plan_create(3, 1, 2, 3, cfg.grid, cfg.modes, "f32", 0)
    try:
        run_layer(3, 1, 2, 3, cfg.grid, cfg.modes, "f32", inp["x"], inp["w"], plan=plan)
        xh = read_spectra(plan, 0).reshape(1, 2, 8, 12, 3)
        ref = oracle.forward3d(inp["x64"], *cfg.modes) / (16 * 32 * 16)
        assert rel_l2(xh, ref) <= 1e-6
    finally:
        fno.fno_plan_destroy(plan)


def test_deterministic_bitwise():
    cfg = wl.CONFIGS["c0"]
    inp = wl.layer_inputs(cfg, "f32")
    a, _ = run_layer(2, 2, 4, 4, cfg.grid, cfg.modes, "f32", inp["x"], inp["w"])
    b, _ = run_layer(2, 2, 4, 4, cfg.grid, cfg.modes, "f32", inp["x"], inp["w"])
    assert np.array_equal(a, b)


def _names(plan):
    return [fno.fno_plan_launch_name(plan, i) for i in range(fno.fno_plan_num_launches(plan))]


def test_launch_structure():
    p2 = fno.fno_plan_create(2, 2, 4, 4, (16, 16), (4, 4), "f32", 0)
    p3 = fno.fno_plan_create(3, 1, 2, 2, (8, 8, 8), (2, 2, 2), "f32", 0)
    try:
        # three launches by default; one on request where a variant exists
        assert fno.fno_plan_get_launch_shape(p2) == "separate"
        assert _names(p2) == ["fno_fwd_plane", "fno_contract", "fno_inv_plane"]
        fno.fno_plan_set_launch_shape(p2, "fused")
        assert _names(p2) == ["fno_layer_fused"]
        p4 = fno.fno_plan_create(2, 1, 2, 2, (128, 128), (16, 16), "f16", 0)
        assert fno.fno_plan_launch_name(p4, 0) == "fno_fwd_plane_mx"
        assert fno.fno_plan_launch_name(p4, 2) == "fno_inv_plane_mx"
        fno.fno_plan_set_launch_shape(p4, "fused")
        assert _names(p4) == ["fno_layer_fused_mx"]
        fno.fno_plan_destroy(p4)
        # no single-launch variant for 256-wide planes
        p5 = fno.fno_plan_create(2, 1, 2, 2, (256, 256), (16, 16), "f16", 0)
        with pytest.raises(fno.FnoError):
            fno.fno_plan_set_launch_shape(p5, "fused")
        fno.fno_plan_destroy(p5)
        assert fno.fno_plan_num_launches(p3) == 5
        with pytest.raises(fno.FnoError):
            fno.fno_plan_set_launch_shape(p3, "fused")  # no single launch in 3D
        assert fno.fno_plan_workspace_bytes(p2) > 0
    finally:
        fno.fno_plan_destroy(p2)
        fno.fno_plan_destroy(p3)


def test_execution_argument_errors():
    import torch
    plan = fno.fno_plan_create(2, 2, 4, 4, (16, 16), (4, 4), "f32", 0)
    L = fno.lib()
    try:
        x = torch.zeros((2 * 4 * 16 * 16 + 64,), device="cuda:0")
        y = torch.zeros((2 * 4 * 16 * 16 + 64,), device="cuda:0")
        w = torch.zeros((8 * 4 * 4 * 4 * 2,), device="cuda:0")
        xp, yp, wp = x.data_ptr(), y.data_ptr(), w.data_ptr()
        s = torch.cuda.current_stream().cuda_stream
        assert L.fno_spectral_conv2d(plan.handle, xp + 4, wp, yp, s) == 1   # misaligned
        assert L.fno_spectral_conv2d(plan.handle, xp, wp, xp + 64, s) == 1  # x / y overlap
        assert L.fno_spectral_conv2d(plan.handle, xp, None, yp, s) == 1     # NULL
        assert L.fno_spectral_conv3d(plan.handle, xp, wp, yp, s) == 1       # wrong ndim
        assert L.fno_plan_run_launch(plan.handle, 7, xp, wp, yp, s) == 1    # bad index
        assert L.fno_spectral_conv2d(plan.handle, xp, wp, yp, s) == 0
        torch.cuda.synchronize()
    finally:
        fno.fno_plan_destroy(plan)


def test_plan_device_out_of_range():
    h = ctypes.c_void_p()
    g = (ctypes.c_int * 2)(16, 16)
    m = (ctypes.c_int * 2)(4, 4)
    assert fno.lib().fno_plan_create(ctypes.byref(h), 2, 1, 1, 1, g, m, 0, 1000) == 1


def test_binding_rejects_wrong_tensors():
    import torch
    plan = fno.fno_plan_create(2, 2, 4, 4, (16, 16), (4, 4), "f16", 0)
    try:
        x = torch.zeros(plan.x_shape(), dtype=torch.float32, device="cuda:0")
        w = torch.zeros(plan.w_shape(), dtype=torch.float16, device="cuda:0")
        y = torch.zeros(plan.y_shape(), dtype=torch.float16, device="cuda:0")
        with pytest.raises(ValueError):
            fno.fno_spectral_conv2d(plan, x, w, y)
        with pytest.raises(ValueError):
            fno.fno_spectral_conv2d(plan, x.half()[:1], w, y)
        fno.fno_spectral_conv2d(plan, to_device(np.zeros(plan.x_shape(), np.float16), "f16"), w, y)
        torch.cuda.synchronize()
        assert float(y.float().abs().max()) == 0.0
    finally:
        fno.fno_plan_destroy(plan)
