"""Float64 full FNO2d forward (CPU) as a composition of plain operations.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The network is the "FNO module" the TurboFNO write-up (sections 1 and 4.3)
drops the fused layer into: lift the per-pixel features with a Linear layer,
a stack of blocks each adding a spectral convolution to a pointwise 1x1
convolution (with bias) and applying GELU, then a two-Linear projection with
GELU between them. GELU is the exact erf form 0.5 x (1 + erf(x / sqrt 2)).
"""

import numpy as np
from scipy.special import erf

from .spectral import spectral_conv2d


def gelu(x: np.ndarray) -> np.ndarray:
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def _pointwise(A: np.ndarray, v: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """out[b, o, h, w] = sum_i A[o, i] v[b, i, h, w] + bias[o]."""
    B, C, H, W = v.shape
    out = np.matmul(A, v.reshape(B, C, H * W))
    out += bias[None, :, None]
    return out.reshape(B, A.shape[0], H, W)


def fno_block2d(v: np.ndarray, spectral: np.ndarray, W: np.ndarray,
                b, m1: int, m2: int, act: bool = True) -> np.ndarray:
    """One block of the module: act(spectral_conv2d(v) + W v + b), act the
    exact GELU or the identity; spectral (2*m1, m2, Ci, Co) complex, W (Co, Ci),
    b (Co,) or None (zero)."""
    bias = np.zeros(W.shape[0]) if b is None else b
    u = spectral_conv2d(v, spectral, m1, m2) + _pointwise(W, v, bias)
    return gelu(u) if act else u


def fno2d_forward(features: np.ndarray, P: np.ndarray, p: np.ndarray,
                  layers: list, Q1: np.ndarray, q1: np.ndarray,
                  Q2: np.ndarray, q2: np.ndarray, m1: int, m2: int):
    """features: (B, 3, H, W); layers: list of dicts with complex
    ``spectral`` (2*m1, m2, C, C), ``W`` (C, C), ``b`` (C,).
    Returns (B, out, H, W) float64."""
    v = _pointwise(P, features, p)
    for layer in layers:
        v = fno_block2d(v, layer["spectral"], layer["W"], layer["b"], m1, m2)
    h = gelu(_pointwise(Q1, v, q1))
    return _pointwise(Q2, h, q2)
