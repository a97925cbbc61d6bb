"""The erf approximation of the half-precision GELU (Abramowitz & Stegun,
Handbook of Mathematical Functions, formula 7.1.28) evaluated step by step
in float32 the way the kernels do, against the exact erf: its absolute
error stays far below the fp16 / bf16 output rounding."""

import math

import numpy as np

A = [0.0705230784, 0.0422820123, 0.0092705272, 0.0001520143, 0.0002765672, 0.0000430638]


def _gelu_f32(v):
    f = np.float32
    v = np.asarray(v, dtype=np.float32)
    x = (np.abs(v) * f(0.70710678118654752)).astype(np.float32)
    p = np.full_like(x, f(A[5]))
    for c in A[4::-1]:
        p = (p * x + f(c)).astype(np.float32)
    p = (p * x + f(1)).astype(np.float32)
    with np.errstate(over="ignore"):
        for _ in range(4):
            p = (p * p).astype(np.float32)
    r = (f(1) / p).astype(np.float32)
    return (np.maximum(v, f(0)) - f(0.5) * np.abs(v) * r).astype(np.float32), r


def test_erf_error_below_2e_6():
    x = np.linspace(0.0, 8.0, 200001)
    _, r = _gelu_f32(x * math.sqrt(2.0))
    ref = np.array([math.erfc(t) for t in x])
    assert np.abs(r.astype(np.float64) - ref).max() < 2e-6


def test_gelu_matches_exact_form():
    v = np.linspace(-12.0, 12.0, 100001)
    g, _ = _gelu_f32(v)
    ref = np.array([0.5 * t * (1.0 + math.erf(t / math.sqrt(2.0))) for t in v])
    # |error| <= |v| / 2 * |erf error| (+ fp32 rounding): about 1e-6 |v|,
    # against an fp16 output rounding of 2^-11 |GELU(v)|
    err = np.abs(g.astype(np.float64) - ref)
    assert (err <= 1.5e-6 * np.maximum(1.0, np.abs(v))).all()
    pos = v > 0.5
    assert (err[pos] / ref[pos]).max() < 1e-5
    # saturation far out: ~0 on the left, the identity on the right
    assert abs(g[0]) < 1e-20
    assert g[-1] == np.float32(12.0)
