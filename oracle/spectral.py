"""Float64 definition of the FNO spectral-convolution layer (CPU, plain numpy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer, as the TurboFNO write-up ("TurboFNO: FFT-GEMM-iFFT fusion
kernels", sections 1, 2.1-2.3) describes the PyTorch pipeline it fuses:
rfft2 of a [B, C, H, W] field, keep the low-frequency mode corners, multiply
each retained mode by a complex C_in x C_out weight summed over the input
channel (section 2.2's einsum "xyij,xyik->xyjk"), zero the rest, irfft2.

Readings of points the pages leave open:
  * normalisation: the default of the named torch.fft pipeline ("backward"):
    forward unnormalised, inverse scaled by 1/(H*W) (1/(X*Y*Z) in 3D);
  * sign: forward exp(-2 pi i k n / N), inverse exp(+2 pi i k n / N);
  * retained modes: kx in [0, m1) and [H-m1, H) (two corners), ky in [0, m2)
    (half spectrum); in 3D the corners are in kx and ky, kz in [0, m3);
  * contraction: no conjugation, a separate weight per retained mode;
  * c2r convention: the inverse keeps the real part of the ky = 0 (kz = 0)
    term and doubles ky >= 1 (numpy / pocketfft irfft semantics); the
    Nyquist bin is never retained because m2 <= W/2.

Each stage is the plain definition written as a dense DFT matrix whose phase
is reduced modulo N in integers before cos/sin are taken in float64.
"""

import numpy as np

TWO_PI = 2.0 * np.pi


def corner_indices(n: int, m: int) -> np.ndarray:
    """Retained indices along a corner axis: [0, m) then [n - m, n)."""
    return np.concatenate([np.arange(m), np.arange(n - m, n)])


def _dft_rows(n: int, ks: np.ndarray, sign: int):
    """cos and sin parts of E[k, t] = exp(sign * 2 pi i * k * t / n)."""
    t = np.arange(n)
    phase = (np.outer(np.asarray(ks, dtype=np.int64), t) % n) * (TWO_PI / n)
    return np.cos(phase), sign * np.sin(phase)


def _real_times_complex_last(x: np.ndarray, c: np.ndarray, s: np.ndarray):
    """sum_t x[..., t] * (c[k, t] + i s[k, t]) for real x, via two real GEMMs."""
    return x @ c.T + 1j * (x @ s.T)


def forward2d(x: np.ndarray, m1: int, m2: int) -> np.ndarray:
    """Truncated 2D forward DFT, unnormalised.

    x: (..., H, W) real. Returns (..., 2*m1, m2) complex with
    out[..., a, ky] = sum_{h,w} x[h, w] exp(-2 pi i (kx h / H + ky w / W)),
    kx = corner_indices(H, m1)[a].
    """
    H, W = x.shape[-2:]
    c, s = _dft_rows(W, np.arange(m2), -1)
    R = _real_times_complex_last(x, c, s)              # (..., H, m2)
    ch, sh = _dft_rows(H, corner_indices(H, m1), -1)
    EH = ch + 1j * sh                                  # (2m1, H)
    return np.einsum("ah,...hy->...ay", EH, R)


def contract(xh: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-mode contraction over the input channel, no conjugation.

    xh: (B, Ci, *modes); w: (*modes, Ci, Co). Returns (B, Co, *modes) with
    out[b, o, k] = sum_i xh[b, i, k] * w[k, i, o].
    """
    B, Ci = xh.shape[:2]
    mshape = xh.shape[2:]
    Co = w.shape[-1]
    K = int(np.prod(mshape))
    a = xh.reshape(B, Ci, K).transpose(2, 0, 1)        # (K, B, Ci)
    b = w.reshape(K, Ci, Co)                           # (K, Ci, Co)
    out = np.matmul(a, b)                              # (K, B, Co)
    return out.transpose(1, 2, 0).reshape((B, Co) + mshape)


def _c2r_last(z: np.ndarray, n: int, m: int) -> np.ndarray:
    """sum_{k<m} g_k Re(z[..., k] exp(+2 pi i k t / n)), g_0 = 1, g_k = 2."""
    g = np.full(m, 2.0)
    g[0] = 1.0
    zg = z * g
    c, s = _dft_rows(n, np.arange(m), +1)              # (m, n)
    return zg.real @ c - zg.imag @ s


def inverse2d(yh: np.ndarray, H: int, W: int, m1: int, m2: int) -> np.ndarray:
    """Closed-form inverse from the retained modes (zero elsewhere).

    yh: (..., 2*m1, m2). Returns (..., H, W) real:
    y[h, w] = 1/(H W) sum_{ky<m2} g_ky Re(Z[h, ky] exp(+2 pi i ky w / W)),
    Z[h, ky] = sum_a yh[a, ky] exp(+2 pi i kx_a h / H).
    """
    ch, sh = _dft_rows(H, corner_indices(H, m1), +1)
    EHi = ch + 1j * sh                                 # (2m1, H)
    Z = np.einsum("ah,...ay->...hy", EHi, yh)          # (..., H, m2)
    return _c2r_last(Z, W, m2) / (H * W)


def spectral_conv2d(x: np.ndarray, w: np.ndarray, m1: int, m2: int):
    """The 2D layer. x: (B, Ci, H, W) float64; w: (2*m1, m2, Ci, Co) complex.
    Returns (B, Co, H, W) float64."""
    H, W = x.shape[-2:]
    return inverse2d(contract(forward2d(x, m1, m2), w), H, W, m1, m2)


def forward3d(x: np.ndarray, m1: int, m2: int, m3: int) -> np.ndarray:
    """Truncated 3D forward DFT, unnormalised: z (half spectrum) then y then x
    (corners). x: (..., X, Y, Z) real -> (..., 2*m1, 2*m2, m3) complex."""
    X, Y, Z = x.shape[-3:]
    c, s = _dft_rows(Z, np.arange(m3), -1)
    R = _real_times_complex_last(x, c, s)              # (..., X, Y, m3)
    cy, sy = _dft_rows(Y, corner_indices(Y, m2), -1)
    R = np.einsum("by,...xyz->...xbz", cy + 1j * sy, R)  # (..., X, 2m2, m3)
    cx, sx = _dft_rows(X, corner_indices(X, m1), -1)
    return np.einsum("ax,...xbz->...abz", cx + 1j * sx, R)


def inverse3d(yh: np.ndarray, X: int, Y: int, Z: int, m1: int, m2: int,
              m3: int) -> np.ndarray:
    """Closed-form 3D inverse: x then y (corners, complex), then the c2r sum
    along z; scaled by 1/(X Y Z). yh: (..., 2*m1, 2*m2, m3)."""
    cx, sx = _dft_rows(X, corner_indices(X, m1), +1)
    T = np.einsum("ax,...abz->...xbz", cx + 1j * sx, yh)  # (..., X, 2m2, m3)
    cy, sy = _dft_rows(Y, corner_indices(Y, m2), +1)
    T = np.einsum("by,...xbz->...xyz", cy + 1j * sy, T)   # (..., X, Y, m3)
    return _c2r_last(T, Z, m3) / (X * Y * Z)


def spectral_conv3d(x: np.ndarray, w: np.ndarray, m1: int, m2: int, m3: int):
    """The 3D layer. x: (B, Ci, X, Y, Z) float64; w: (2*m1, 2*m2, m3, Ci, Co)
    complex. Returns (B, Co, X, Y, Z) float64."""
    X, Y, Z = x.shape[-3:]
    return inverse3d(contract(forward3d(x, m1, m2, m3), w), X, Y, Z, m1, m2, m3)
