"""GPU parity of the full FNO2d network and its per-pixel kernels against the
float64 oracle (relative L2 <= 3e-3 for fp16 storage, 1e-5 for fp32)."""

import numpy as np
import pytest

import oracle
import spectral_convolution_amd as fno
import workloads as wl
from gpu_util import rel_l2, to_device, to_float64

pytestmark = pytest.mark.gpu


def _rand(rng, shape, dtype, scale=1.0):
    v = rng.standard_normal(shape) * scale
    s = wl.round_to_storage(v, dtype)
    return s, wl.storage_to_float64(s, dtype)


@pytest.mark.parametrize("dtype,B,I,O,P,act,add", [
    ("f32", 2, 3, 64, 4096, 0, False),     # lift shape
    ("f16", 3, 64, 64, 1000, 1, True),     # block epilogue, ragged pixel count
    ("bf16", 1, 17, 70, 259, 1, True),     # ragged channels (two output blocks)
    ("f32", 2, 128, 5, 64, 0, False),
    # fp16 / bf16 with P % 8 == 0 run on half-precision matrix cores
    ("f16", 2, 3, 64, 4096, 0, False),     # lift shape, one 32-channel block
    ("bf16", 2, 64, 64, 2048, 1, True),    # block epilogue, two blocks
    ("f16", 1, 60, 70, 520, 1, True),      # two blocks, ragged outputs, half-tile tail (P % 16 == 8)
    ("bf16", 3, 33, 5, 8, 0, True),        # one pixel group per batch element
    ("f16", 1, 128, 130, 768, 1, False),   # over 64 inputs: the fp32-operand kernel
])
def test_channel_mix(dtype, B, I, O, P, act, add):
    import torch
    rng = np.random.default_rng(5)
    xs, x64 = _rand(rng, (B, I, P), dtype)
    As, A64 = _rand(rng, (O, I), dtype, 1 / np.sqrt(I))
    bs, b64 = _rand(rng, (O,), dtype)
    ads, ad64 = _rand(rng, (B, O, P), dtype)
    x, A, b = to_device(xs, dtype), to_device(As, dtype), to_device(bs, dtype)
    ad = to_device(ads, dtype) if add else None
    y = torch.empty((B, O, P), dtype=x.dtype, device=x.device)
    fno.fno_channel_mix(x, A, b, ad, y, act)
    torch.cuda.synchronize()
    ref = np.einsum("oi,bip->bop", A64, x64) + b64[None, :, None] + (ad64 if add else 0)
    if act:
        ref = oracle.gelu(ref)
    tol = 1e-5 if dtype == "f32" else 3e-3
    assert rel_l2(to_float64(y), ref) <= tol


@pytest.mark.parametrize("dtype,B,I,J,C,P", [
    ("f16", 2, 64, 128, 1, 4096),
    ("f32", 1, 20, 33, 3, 333),
    # fp16 / bf16 with P % 8 == 0 run on half-precision matrix cores
    ("bf16", 2, 33, 100, 4, 520),   # two input blocks, ragged hidden units, four outputs
    ("f16", 3, 20, 128, 2, 8),      # one pixel group per batch element
    ("bf16", 1, 64, 128, 1, 4096),  # the network's shape
])
def test_projection(dtype, B, I, J, C, P):
    import torch
    rng = np.random.default_rng(6)
    xs, x64 = _rand(rng, (B, I, P), dtype)
    Q1s, Q164 = _rand(rng, (J, I), dtype, 1 / np.sqrt(I))
    q1s, q164 = _rand(rng, (J,), dtype)
    Q2s, Q264 = _rand(rng, (C, J), dtype, 1 / np.sqrt(J))
    q2s, q264 = _rand(rng, (C,), dtype)
    t = [to_device(v, dtype) for v in (xs, Q1s, q1s, Q2s, q2s)]
    y = torch.empty((B, C, P), dtype=t[0].dtype, device=t[0].device)
    fno.fno_projection(*t, y)
    torch.cuda.synchronize()
    h = oracle.gelu(np.einsum("ji,bip->bjp", Q164, x64) + q164[None, :, None])
    ref = np.einsum("cj,bjp->bcp", Q264, h) + q264[None, :, None]
    tol = 1e-5 if dtype == "f32" else 3e-3
    assert rel_l2(to_float64(y), ref) <= tol


def _run_model(cfg, batch=None, grid=None, samples=None, spectral_scale=None, n_layers=None):
    import torch
    inp = wl.model_inputs(cfg, batch=batch, grid=grid)
    if n_layers is not None:
        inp["layers"], inp["layers64"] = inp["layers"][:n_layers], inp["layers64"][:n_layers]
    nl = len(inp["layers"])
    dt = inp["dtype"]
    if spectral_scale is not None:
        # stronger spectral weights, re-rounded to storage; the oracle gets
        # the stored values
        for L, L64 in zip(inp["layers"], inp["layers64"]):
            s = wl.round_to_storage(wl.storage_to_float64(L["spectral"], dt) * spectral_scale, dt)
            L["spectral"] = s
            v = wl.storage_to_float64(s, dt)
            L64["spectral"] = v[..., 0] + 1j * v[..., 1]
    B = inp["batch"]
    H, W = inp["grid"]
    model = fno.fno_model2d_create(B, (H, W), cfg.in_channels, cfg.width, nl, cfg.modes,
                                   cfg.proj_hidden, cfg.out_channels, dt, 0)
    try:
        params = [to_device(inp["P"], dt), to_device(inp["p"], dt)]
        for L in inp["layers"]:
            params += [to_device(L["spectral"], dt), to_device(L["W"], dt), to_device(L["b"], dt)]
        params += [to_device(inp[k], dt) for k in ("Q1", "q1", "Q2", "q2")]
        f = to_device(inp["features"], dt)
        out = torch.empty((B, cfg.out_channels, H, W), dtype=f.dtype, device=f.device)
        fno.fno_model2d_forward(model, f, params, out)
        torch.cuda.synchronize()
        got = to_float64(out)
    finally:
        fno.fno_model2d_destroy(model)
    idx = list(range(B)) if samples is None else list(samples)
    ref = oracle.fno2d_forward(inp["features64"][idx], inp["P64"], inp["p64"], inp["layers64"],
                               inp["Q164"], inp["q164"], inp["Q264"], inp["q264"], *cfg.modes)
    return got[idx], ref


def test_model_small():
    cfg = wl.CONFIGS["c4"]
    got, ref = _run_model(cfg, batch=2, grid=(64, 64))
    err = rel_l2(got, ref)
    print(f"[model] 64x64 B=2 rel_l2={err:.3e}", flush=True)
    assert err <= 3e-3


def test_model_full_size_sampled():
    cfg = wl.CONFIGS["c4"]
    print("[model-full] B=20 256x256 samples (0, 19)", flush=True)
    got, ref = _run_model(cfg, samples=(0, 19))
    err = rel_l2(got, ref)
    print(f"[model-full] rel_l2={err:.3e}", flush=True)
    assert err <= 3e-3


def test_model_spectral_branch_weighted():
    """With the workload's spectral weights ((1/64^2) U[0,1)) the spectral
    branch is ~1e-4 of the output norm, below the tolerance; scaled by 512
    it is ~77 %, so an error in the spectral layers inside the model shows."""
    cfg = wl.CONFIGS["c4"]
    got, ref = _run_model(cfg, batch=2, grid=(64, 64), spectral_scale=512.0)
    err = rel_l2(got, ref)
    print(f"[model] 64x64 B=2 spectral x512 rel_l2={err:.3e}", flush=True)
    assert err <= 3e-3



def test_model_full_size_spectral_branch_weighted():
    """The B=20, 256x256 network with its spectral weights scaled by 512, so
    that the spectral branch carries most of the output (the workload's own
    weights leave it ~1e-4 of the output norm); sampled batch elements."""
    cfg = wl.CONFIGS["c4"]
    print("[model-full] B=20 256x256 spectral x512 samples (0, 19)", flush=True)
    got, ref = _run_model(cfg, samples=(0, 19), spectral_scale=512.0)
    err = rel_l2(got, ref)
    print(f"[model-full] spectral x512 rel_l2={err:.3e}", flush=True)
    assert err <= 3e-3


def test_model_without_blocks():
    # no blocks: the lift is not folded anywhere and runs as its own kernel
    cfg = wl.CONFIGS["c4"]
    got, ref = _run_model(cfg, batch=2, grid=(64, 64), n_layers=0)
    assert rel_l2(got, ref) <= 3e-3


def test_model_graph_replay_matches_eager():
    """Graph replay of the forward equals the eager forward bit for bit, on
    every replay, with eager work between replays; new pointers re-capture."""
    import torch
    cfg = wl.CONFIGS["c4"]
    inp = wl.model_inputs(cfg, batch=2, grid=(64, 64))
    dt = inp["dtype"]
    model = fno.fno_model2d_create(2, (64, 64), cfg.in_channels, cfg.width, cfg.n_layers, cfg.modes,
                                   cfg.proj_hidden, cfg.out_channels, dt, 0)
    try:
        params = [to_device(inp["P"], dt), to_device(inp["p"], dt)]
        for L in inp["layers"]:
            params += [to_device(L["spectral"], dt), to_device(L["W"], dt), to_device(L["b"], dt)]
        params += [to_device(inp[k], dt) for k in ("Q1", "q1", "Q2", "q2")]
        f = to_device(inp["features"], dt)
        ref = torch.empty((2, 1, 64, 64), dtype=f.dtype, device=f.device)
        fno.fno_model2d_forward(model, f, params, ref)
        torch.cuda.synchronize()
        fno.fno_model2d_set_graph(model, True)
        outs = [torch.empty_like(ref), torch.empty_like(ref)]
        for rep in range(4):
            out = outs[rep // 2]  # the second pointer forces a new capture
            out.zero_()
            torch.cuda.synchronize()
            fno.fno_model2d_forward(model, f, params, out)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), f"replay {rep} differs from the eager forward"
            # eager work between replays
            fno.fno_model2d_set_graph(model, False)
            fno.fno_model2d_forward(model, f, params, torch.empty_like(ref))
            fno.fno_model2d_set_graph(model, True)
            torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        fno.fno_model2d_destroy(model)
