"""GPU parity of fno_block2d, one FNO block y = act(spectral conv + 1x1 + bias)
with the spectral branch finished in the row-stage epilogue, against the
float64 oracle block (relative L2 <= 3e-3 for fp16 / bf16 storage). Each
branch is also checked alone against the library's own stand-alone layer
and channel mix, so that a wrong spectral branch cannot hide under the 1x1
branch or the other way round."""

import numpy as np
import pytest

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu

TOL = 3e-3


def _rand(rng, shape, dtype, scale=1.0):
    s = wl.round_to_storage(rng.standard_normal(shape) * scale, dtype)
    return s, wl.storage_to_float64(s, dtype)


def _case(dtype, B, Ci, Co, H, W, m1, m2, seed):
    rng = np.random.default_rng(seed)
    xs, x64 = _rand(rng, (B, Ci, H, W), dtype)
    # spectral weights large enough that the spectral branch carries a share
    # of the output comparable to the 1x1 branch
    wc = (rng.standard_normal((2 * m1, m2, Ci, Co)) + 1j * rng.standard_normal((2 * m1, m2, Ci, Co))) * (
        4.0 / np.sqrt(Ci))
    ws = wl.round_to_storage(wl.complex_to_interleaved(wc), dtype)
    w64i = wl.storage_to_float64(ws, dtype)
    w64 = w64i[..., 0] + 1j * w64i[..., 1]
    As, A64 = _rand(rng, (Co, Ci), dtype, 1.0 / np.sqrt(Ci))
    bs, b64 = _rand(rng, (Co,), dtype, 0.5)
    return xs, x64, ws, w64, As, A64, bs, b64


CASES = [
    # dtype, B, Ci, Co, H, W, m1, m2, act, bias
    ("f16", 2, 64, 64, 64, 64, 24, 24, 1, True),     # the network's block shape, small grid
    ("f16", 2, 3, 64, 128, 128, 16, 16, 1, True),    # first block on 3 feature channels (one k-block)
    ("bf16", 1, 64, 68, 64, 128, 20, 24, 1, False),  # two output blocks (ragged), no bias
    ("f16", 3, 33, 20, 256, 256, 24, 24, 0, True),   # no act, ragged inputs over one k-block, 4 waves
    ("bf16", 2, 32, 64, 64, 64, 5, 7, 1, True),      # small ragged modes (one ky tile)
    ("f16", 1, 64, 64, 256, 256, 32, 32, 1, True),   # full 2 x 16 ky tiles, 64-wide Z rows
    # batch 16: the spectra travel as the half exchange (fp16 pairs + exponents)
    ("f16", 16, 64, 64, 64, 64, 24, 24, 1, True),
    ("bf16", 16, 3, 64, 128, 128, 24, 24, 1, True),
]
HALF_EXCHANGE = {16}


@pytest.mark.parametrize("dtype,B,Ci,Co,H,W,m1,m2,act,bias", CASES)
def test_block_vs_oracle(dtype, B, Ci, Co, H, W, m1, m2, act, bias):
    import torch
    xs, x64, ws, w64, As, A64, bs, b64 = _case(dtype, B, Ci, Co, H, W, m1, m2, 3)
    print(f"block {dtype} B={B} {Ci}->{Co} {H}x{W} modes {m1}x{m2} act={act}", flush=True)
    plan = fno.fno_plan_create(2, B, Ci, Co, (H, W), (m1, m2), dtype, 0)
    try:
        assert fno.fno_plan_spectra_format(plan) == (1 if B in HALF_EXCHANGE else 0)
        x, w, A = to_device(xs, dtype), to_device(ws, dtype), to_device(As, dtype)
        b = to_device(bs, dtype) if bias else None
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        fno.fno_block2d(plan, x, w, A, b, y, act)
        torch.cuda.synchronize()
        ref = oracle.fno_block2d(x64, w64, A64, b64 if bias else None, m1, m2, act=bool(act))
        err = rel_l2(to_float64(y), ref)
        assert err <= TOL, err
        # a second call on the same buffers gives the same bits
        y2 = torch.empty_like(y)
        fno.fno_block2d(plan, x, w, A, b, y2, act)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    finally:
        fno.fno_plan_destroy(plan)


@pytest.mark.parametrize("dtype,B,Ci,Co,H,W,m1,m2", [
    ("f16", 2, 64, 64, 64, 64, 24, 24),
    ("bf16", 1, 3, 64, 128, 128, 16, 16),
])
def test_block_branches_alone(dtype, B, Ci, Co, H, W, m1, m2):
    """Zero 1x1 weights and no act: the spectral layer's own output; zero
    spectral weights: the channel mix's."""
    import torch
    xs, x64, ws, w64, As, A64, bs, b64 = _case(dtype, B, Ci, Co, H, W, m1, m2, 4)
    plan = fno.fno_plan_create(2, B, Ci, Co, (H, W), (m1, m2), dtype, 0)
    try:
        x, w, A, b = to_device(xs, dtype), to_device(ws, dtype), to_device(As, dtype), to_device(bs, dtype)
        y = torch.empty(plan.y_shape(), dtype=x.dtype, device=x.device)
        ys = torch.empty_like(y)
        fno.fno_block2d(plan, x, w, torch.zeros_like(A), None, y, 0)
        fno.fno_spectral_conv2d(plan, x, w, ys)
        torch.cuda.synchronize()
        a, r = to_float64(y), to_float64(ys)
        assert rel_l2(a, r) <= 2e-3
        fno.fno_block2d(plan, x, torch.zeros_like(w), A, b, y, 1)
        ym = torch.empty_like(y)
        fno.fno_channel_mix(x, A, b, None, ym, 1)
        torch.cuda.synchronize()
        assert rel_l2(to_float64(y), to_float64(ym)) <= 2e-3
    finally:
        fno.fno_plan_destroy(plan)


def test_block_unsupported_plans():
    import torch
    # fp32 storage (no half exchange) and more than 64 input channels
    for dtype, Ci in (("f32", 8), ("f16", 65)):
        plan = fno.fno_plan_create(2, 1, Ci, 8, (64, 64), (4, 4), dtype, 0)
        try:
            td = torch.float32 if dtype == "f32" else torch.float16
            x = torch.zeros(plan.x_shape(), dtype=td, device="cuda")
            w = torch.zeros(plan.w_shape(), dtype=td, device="cuda")
            A = torch.zeros((8, Ci), dtype=td, device="cuda")
            y = torch.empty(plan.y_shape(), dtype=td, device="cuda")
            with pytest.raises(fno.FnoError) as e:
                fno.fno_block2d(plan, x, w, A, None, y, 1)
            assert e.value.status == 2  # FNO_ERR_UNSUPPORTED
            with pytest.raises(fno.FnoError):
                fno.fno_block2d_prepare(plan)
        finally:
            fno.fno_plan_destroy(plan)
