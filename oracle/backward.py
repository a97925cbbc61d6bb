"""Float64 gradients of the spectral-convolution layer (CPU, plain numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer is y = C(contract(F x, w)): F is the truncated forward DFT (the
rfft2 / rfftn of the TurboFNO write-up's section 2.1 pipeline, kept modes
only, unnormalised), contract is section 2.2's per-mode weight einsum, and C
is the closed-form inverse (irfft2 / irfftn of the zero-filled spectrum,
scaled by 1/N). Section 4.3 of the write-up exposes the layer to PyTorch
autograd through a backward function; what that backward must return is
fixed by the forward alone. For a loss with gradient g = dL/dy, every step
is linear, so the gradients are the adjoints of the steps applied in
reverse order:

  Gh = C^T g          C^T g [k] = (gamma_k / N) (F g)[k]
  dw[k][i][o]       = sum_b conj(Xh[b, i, k]) Gh[b, o, k],   Xh = F x
  dXh[b, i, k]      = sum_o Gh[b, o, k] conj(w[k][i][o])
  dx = F^T dXh        F^T z [n] = Re sum_k z[k] exp(+2 pi i k.n / N)

Complex quantities are pairs of reals with the inner product Re(conj(a) b);
the gradient of a complex weight is dL/dRe(w) + i dL/dIm(w) (the convention
of PyTorch autograd). gamma_k is the c2r weight of the last-axis mode: 1 for
index 0 (only its real part reaches y), 2 otherwise. N = H W (2D) or X Y Z
(3D).
"""

import numpy as np

from .spectral import _dft_rows, contract, corner_indices, forward2d, forward3d


def _gamma(m: int) -> np.ndarray:
    g = np.full(m, 2.0)
    g[0] = 1.0
    return g


def adjoint_inverse2d(g: np.ndarray, m1: int, m2: int) -> np.ndarray:
    """C^T for the 2D inverse: g (..., H, W) real -> (..., 2*m1, m2) complex,
    out[a, ky] = (gamma_ky / (H W)) sum_{h,w} g[h, w] exp(-2 pi i (kx_a h / H + ky w / W))."""
    H, W = g.shape[-2:]
    return forward2d(g, m1, m2) * (_gamma(m2) / (H * W))


def adjoint_forward2d(z: np.ndarray, H: int, W: int, m1: int, m2: int) -> np.ndarray:
    """F^T for the truncated 2D forward DFT: z (..., 2*m1, m2) complex ->
    (..., H, W) real, out[h, w] = Re sum_{a,ky} z[a, ky] exp(+2 pi i (kx_a h / H + ky w / W))."""
    ch, sh = _dft_rows(H, corner_indices(H, m1), +1)
    Zh = np.einsum("ah,...ay->...hy", ch + 1j * sh, z)   # (..., H, m2)
    c, s = _dft_rows(W, np.arange(m2), +1)               # (m2, W)
    return Zh.real @ c - Zh.imag @ s


def adjoint_inverse3d(g: np.ndarray, m1: int, m2: int, m3: int) -> np.ndarray:
    """C^T for the 3D inverse: (gamma_kz / (X Y Z)) times the truncated forward DFT."""
    X, Y, Z = g.shape[-3:]
    return forward3d(g, m1, m2, m3) * (_gamma(m3) / (X * Y * Z))


def adjoint_forward3d(z: np.ndarray, X: int, Y: int, Z: int, m1: int, m2: int,
                      m3: int) -> np.ndarray:
    """F^T for the truncated 3D forward DFT: z (..., 2*m1, 2*m2, m3) ->
    (..., X, Y, Z) real, Re of the sum over retained modes with exp(+...)."""
    cx, sx = _dft_rows(X, corner_indices(X, m1), +1)
    T = np.einsum("ax,...abz->...xbz", cx + 1j * sx, z)   # (..., X, 2m2, m3)
    cy, sy = _dft_rows(Y, corner_indices(Y, m2), +1)
    T = np.einsum("by,...xbz->...xyz", cy + 1j * sy, T)   # (..., X, Y, m3)
    c, s = _dft_rows(Z, np.arange(m3), +1)                # (m3, Z)
    return T.real @ c - T.imag @ s


def contract_adjoint_x(gh: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Adjoint of the contraction in its spectra argument.

    gh: (B, Co, *modes); w: (*modes, Ci, Co). Returns (B, Ci, *modes) with
    out[b, i, k] = sum_o gh[b, o, k] conj(w[k, i, o]), i.e. the contraction
    with the per-mode conjugate transpose of w.
    """
    wh = np.conj(np.swapaxes(w, -1, -2))                 # (*modes, Co, Ci)
    return contract(gh, wh)


def contract_grad_w(xh: np.ndarray, gh: np.ndarray) -> np.ndarray:
    """Gradient of the contraction in its weight argument.

    xh: (B, Ci, *modes), gh: (B, Co, *modes). Returns (*modes, Ci, Co) with
    out[k, i, o] = sum_b conj(xh[b, i, k]) gh[b, o, k].
    """
    B, Ci = xh.shape[:2]
    Co = gh.shape[1]
    mshape = xh.shape[2:]
    K = int(np.prod(mshape))
    a = np.conj(xh.reshape(B, Ci, K)).transpose(2, 1, 0)  # (K, Ci, B)
    b = gh.reshape(B, Co, K).transpose(2, 0, 1)           # (K, B, Co)
    return np.matmul(a, b).reshape(mshape + (Ci, Co))


def spectral_conv2d_backward(x: np.ndarray, w: np.ndarray, g: np.ndarray, m1: int, m2: int):
    """Gradients of the 2D layer. x: (B, Ci, H, W); w: (2*m1, m2, Ci, Co)
    complex; g = dL/dy: (B, Co, H, W). Returns (dx (B, Ci, H, W) float64,
    dw (2*m1, m2, Ci, Co) complex128)."""
    H, W = x.shape[-2:]
    gh = adjoint_inverse2d(g, m1, m2)
    dw = contract_grad_w(forward2d(x, m1, m2), gh)
    dx = adjoint_forward2d(contract_adjoint_x(gh, w), H, W, m1, m2)
    return dx, dw


def spectral_conv3d_backward(x: np.ndarray, w: np.ndarray, g: np.ndarray, m1: int, m2: int,
                             m3: int):
    """Gradients of the 3D layer. x: (B, Ci, X, Y, Z); w: (2*m1, 2*m2, m3,
    Ci, Co) complex; g: (B, Co, X, Y, Z). Returns (dx, dw)."""
    X, Y, Z = x.shape[-3:]
    gh = adjoint_inverse3d(g, m1, m2, m3)
    dw = contract_grad_w(forward3d(x, m1, m2, m3), gh)
    dx = adjoint_forward3d(contract_adjoint_x(gh, w), X, Y, Z, m1, m2, m3)
    return dx, dw
