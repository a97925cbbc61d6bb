"""Pins for the oracle's full FNO2d forward.

With all spectral weights zero the network is a per-pixel MLP, written out
here with explicit loops and math.erf. The end-to-end network with nonzero
spectral weights is a composition of pinned parts (the layer pins in
test_oracle_pins.py plus this test); it has no independent end-to-end value.
"""

import math

import numpy as np

import oracle


def _gelu_scalar(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def test_gelu_values():
    xs = np.array([-3.0, -1.0, -0.25, 0.0, 0.5, 1.0, 2.5])
    got = oracle.gelu(xs)
    ref = np.array([_gelu_scalar(v) for v in xs])
    assert np.abs(got - ref).max() <= 1e-15
    # GELU(1) = Phi(1) = 0.8413447460685429 (standard normal CDF at 1)
    assert abs(oracle.gelu(np.array([1.0]))[0] - 0.8413447460685429) <= 1e-15


def test_zero_spectral_weights_is_pixel_mlp():
    rng = np.random.default_rng(7)
    B, H, W, C, hid, m1, m2 = 2, 8, 8, 4, 6, 2, 3
    f = rng.standard_normal((B, 3, H, W))
    P, p = rng.standard_normal((C, 3)), rng.standard_normal(C)
    layers = []
    for _ in range(2):
        layers.append({"spectral": np.zeros((2 * m1, m2, C, C), dtype=np.complex128),
                       "W": rng.standard_normal((C, C)) * 0.5,
                       "b": rng.standard_normal(C)})
    Q1, q1 = rng.standard_normal((hid, C)), rng.standard_normal(hid)
    Q2, q2 = rng.standard_normal((1, hid)), rng.standard_normal(1)
    got = oracle.fno2d_forward(f, P, p, layers, Q1, q1, Q2, q2, m1, m2)

    ref = np.zeros((B, 1, H, W))
    for b in range(B):
        for h in range(H):
            for w in range(W):
                v = [sum(P[o, c] * f[b, c, h, w] for c in range(3)) + p[o] for o in range(C)]
                for L in layers:
                    v = [_gelu_scalar(sum(L["W"][o, i] * v[i] for i in range(C)) + L["b"][o])
                         for o in range(C)]
                t = [_gelu_scalar(sum(Q1[j, i] * v[i] for i in range(C)) + q1[j]) for j in range(hid)]
                ref[b, 0, h, w] = sum(Q2[0, j] * t[j] for j in range(hid)) + q2[0]
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())


def test_spectral_branch_is_added_before_gelu():
    # one block, zero bypass: v1 = GELU(SpecConv(v0)); with identity spectral
    # weights on a single sinusoid that the layer passes unchanged, the block
    # output is GELU of the lifted sinusoid itself.
    H = W = 16
    m1 = m2 = 4
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    s = np.cos(2 * np.pi * (2 * hh / H + 1 * ww / W))
    f = np.zeros((1, 3, H, W))
    f[0, 0] = s
    C = 2
    P = np.zeros((C, 3))
    P[0, 0], P[1, 0] = 1.0, -0.5
    p = np.zeros(C)
    spec = np.zeros((2 * m1, m2, C, C), dtype=np.complex128)
    spec[..., 0, 0] = spec[..., 1, 1] = 1.0
    layers = [{"spectral": spec, "W": np.zeros((C, C)), "b": np.zeros(C)}]
    Q1 = np.eye(C)
    q1 = np.zeros(C)
    Q2 = np.array([[1.0, 0.0]])
    q2 = np.zeros(1)
    got = oracle.fno2d_forward(f, P, p, layers, Q1, q1, Q2, q2, m1, m2)
    g = np.vectorize(_gelu_scalar)
    ref = g(g(s))
    assert np.abs(got[0, 0] - ref).max() <= 1e-13


def test_block_is_spectral_plus_pointwise():
    # fno_block2d without act: a sinusoid the layer passes unchanged (identity
    # spectral weights on channel 0, zero elsewhere) plus the 1x1 convolution
    # and bias written with loops; with act, GELU of that, and a None bias is
    # a zero bias.
    H = W = 16
    m1 = m2 = 4
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    rng = np.random.default_rng(11)
    Ci, Co = 2, 3
    v = np.zeros((1, Ci, H, W))
    v[0, 0] = np.cos(2 * np.pi * (1 * hh / H + 3 * ww / W))
    v[0, 1] = rng.standard_normal((H, W))
    spec = np.zeros((2 * m1, m2, Ci, Co), dtype=np.complex128)
    spec[..., 0, 0] = 1.0
    Wb = rng.standard_normal((Co, Ci))
    b = rng.standard_normal(Co)
    got = oracle.fno_block2d(v, spec, Wb, b, m1, m2, act=False)
    ref = np.zeros((1, Co, H, W))
    for o in range(Co):
        for h in range(H):
            for w in range(W):
                ref[0, o, h, w] = sum(Wb[o, i] * v[0, i, h, w] for i in range(Ci)) + b[o]
    ref[0, 0] += v[0, 0]
    assert np.abs(got - ref).max() <= 1e-12
    g = np.vectorize(_gelu_scalar)
    assert np.abs(oracle.fno_block2d(v, spec, Wb, b, m1, m2) - g(ref)).max() <= 1e-12
    assert np.abs(oracle.fno_block2d(v, spec, Wb, None, m1, m2, act=False)
                  - (ref - b[None, :, None, None])).max() <= 1e-12
