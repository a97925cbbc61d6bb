"""Pins for the float64 backward oracle: results that mathematics or an
independent library fixes.

* PyTorch CPU autograd (float64) through the torch.fft pipeline the TurboFNO
  write-up names (rfft2 / rfftn, keep the corners, per-mode einsum, zero-fill,
  irfft2 / irfftn): the gradients a user of that pipeline gets.
* The adjoint identities of a layer that is linear in x and in w, against a
  forward written with numpy.fft (not the oracle's DFT matrices):
  <g, L(v, w)> = <dx, v> for any v, and <g, L(x, u)> = Re sum conj(dw) u for
  any u.
* Closed forms: identity weights make the layer the low-pass projection P,
  which is self-adjoint, so dx = P g; a delta input and a cosine gradient
  put dw at the cosine's mode only, with the value gamma / 2 (1/2 on the
  ky = 0 column, where both the mode and its mirror are retained).

Each check takes the backward under test as a callable, so planted mistakes
can be shown to fail them.
"""

import numpy as np

import pins

corners = pins.corners


def numpy_layer2d(x, w, m1, m2):
    """The 2D layer through numpy.fft (rfft2 -> corners -> einsum -> irfft2)."""
    B, Ci, H, W = x.shape
    Co = w.shape[-1]
    X = np.fft.rfft2(x)
    kx = corners(H, m1)
    Y = np.zeros((B, Co, H, W // 2 + 1), dtype=np.complex128)
    Y[:, :, kx, :m2] = np.einsum("biay,ayio->boay", X[:, :, kx, :m2], w)
    return np.fft.irfft2(Y, s=(H, W))


def numpy_layer3d(x, w, m1, m2, m3):
    B, Ci, X, Y, Z = x.shape
    Co = w.shape[-1]
    F = np.fft.rfftn(x, axes=(-3, -2, -1))
    kx, ky = corners(X, m1), corners(Y, m2)
    sel = F[:, :, kx][:, :, :, ky][..., :m3]
    Yf = np.zeros((B, Co, X, Y, Z // 2 + 1), dtype=np.complex128)
    Yf[np.ix_(range(B), range(Co), kx, ky, range(m3))] = np.einsum("nixyz,xyzio->noxyz", sel, w)
    return np.fft.irfftn(Yf, s=(X, Y, Z), axes=(-3, -2, -1))


def _cplx(rng, shape):
    return rng.standard_normal(shape) + 1j * rng.standard_normal(shape)


def _rel(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


def torch_grads(x, w, g, modes):
    """x.grad and w.grad of sum(y * g) by torch CPU autograd, float64."""
    import torch
    nd = len(modes)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.complex128, requires_grad=True)
    gt = torch.tensor(g, dtype=torch.float64)
    dims = tuple(range(-nd, 0))
    grid = x.shape[-nd:]
    F = torch.fft.rfftn(xt, dim=dims)
    B, Co = x.shape[0], w.shape[-1]
    full = torch.zeros((B, Co) + tuple(grid[:-1]) + (grid[-1] // 2 + 1,), dtype=torch.complex128)
    if nd == 2:
        m1, m2 = modes
        kx = torch.tensor(corners(grid[0], m1))
        out = torch.einsum("biay,ayio->boay", F[:, :, kx, :m2], wt)
        full[:, :, kx, :m2] = out
    else:
        m1, m2, m3 = modes
        kx = corners(grid[0], m1)
        ky = corners(grid[1], m2)
        sel = F[:, :, kx][:, :, :, ky][..., :m3]
        out = torch.einsum("nixyz,xyzio->noxyz", sel, wt)
        for a, i in enumerate(kx):
            for b, j in enumerate(ky):
                full[:, :, i, j, :m3] = out[:, :, a, b]
    y = torch.fft.irfftn(full, s=tuple(grid), dim=dims)
    (y * gt).sum().backward()
    return xt.grad.numpy(), wt.grad.numpy()


# ------------------------------------------------------------------------ 2D

def check_backward2d_torch(backward2d, rng):
    for (B, Ci, Co, H, W, m1, m2) in [(2, 3, 4, 16, 16, 4, 4), (1, 2, 3, 16, 32, 5, 7),
                                      (2, 3, 3, 8, 16, 4, 8)]:
        x = rng.standard_normal((B, Ci, H, W))
        w = _cplx(rng, (2 * m1, m2, Ci, Co))
        g = rng.standard_normal((B, Co, H, W))
        dx, dw = backward2d(x, w, g, m1, m2)
        rx, rw = torch_grads(x, w, g, (m1, m2))
        ex, ew = _rel(dx, rx), _rel(dw, rw)
        if not (ex <= 1e-12 and ew <= 1e-12):
            return False, f"torch autograd {H}x{W} m=({m1},{m2}): dx {ex:.2e} dw {ew:.2e}"
    return True, ""


def check_backward2d_adjoint(backward2d, rng):
    B, Ci, Co, H, W, m1, m2 = 2, 3, 3, 16, 32, 5, 6
    x = rng.standard_normal((B, Ci, H, W))
    w = _cplx(rng, (2 * m1, m2, Ci, Co))
    g = rng.standard_normal((B, Co, H, W))
    dx, dw = backward2d(x, w, g, m1, m2)
    for _ in range(3):
        v = rng.standard_normal(x.shape)
        u = _cplx(rng, w.shape)
        lhs_x = float((g * numpy_layer2d(v, w, m1, m2)).sum())
        rhs_x = float((dx * v).sum())
        lhs_w = float((g * numpy_layer2d(x, u, m1, m2)).sum())
        rhs_w = float(np.real(np.conj(dw) * u).sum())
        ex = abs(lhs_x - rhs_x) / (abs(lhs_x) + 1e-300)
        ew = abs(lhs_w - rhs_w) / (abs(lhs_w) + 1e-300)
        if not (ex <= 1e-11 and ew <= 1e-11):
            return False, f"adjoint identity: x {ex:.2e} w {ew:.2e}"
    return True, ""


def check_backward2d_closed_forms(backward2d, rng):
    H, W, m1, m2 = 16, 16, 4, 4
    # identity weights: dx = P g with P the exact low-pass projection
    C = 2
    w = pins.identity_weights((2 * m1, m2), C)
    g = rng.standard_normal((1, C, H, W))
    x = rng.standard_normal((1, C, H, W))
    dx, _ = backward2d(x, w, g, m1, m2)
    M = pins.lowpass_mask2d(H, W, m1, m2)
    ref = np.fft.ifft2(np.fft.fft2(g) * M).real
    e = _rel(dx, ref)
    if not e <= 1e-12:
        return False, f"identity weights: dx vs low-pass of g, err {e:.3e}"
    # delta input, cosine gradient: dw is gamma/2 at the cosine's mode(s)
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    x = np.zeros((1, 1, H, W))
    x[0, 0, 0, 0] = 1.0
    w1 = np.zeros((2 * m1, m2, 1, 1), dtype=np.complex128)
    kxs = corners(H, m1)
    for (p, q) in [(1, 2), (-3, 1), (2, 0), (0, 3), (-2, 0)]:
        g = np.cos(2 * np.pi * (p * hh / H + q * ww / W))[None, None]
        _, dw = backward2d(x, w1, g, m1, m2)
        ref = np.zeros_like(dw)
        for a, kx in enumerate(kxs):
            for ky in range(m2):
                sk = kx if kx < H // 2 else kx - H
                if (sk, ky) == (p, q) or (q == 0 and (sk, ky) == (-p, 0)):
                    ref[a, ky, 0, 0] += 0.5 if q == 0 else 1.0
        if p == 0 and q == 0:
            ref *= 2
        e = np.abs(dw - ref).max()
        if not e <= 1e-13:
            return False, f"delta/cosine ({p},{q}): dw err {e:.3e}"
    return True, ""


# ------------------------------------------------------------------------ 3D

def check_backward3d_torch(backward3d, rng):
    B, Ci, Co, X, Y, Z, m1, m2, m3 = 2, 2, 3, 8, 8, 16, 2, 3, 4
    x = rng.standard_normal((B, Ci, X, Y, Z))
    w = _cplx(rng, (2 * m1, 2 * m2, m3, Ci, Co))
    g = rng.standard_normal((B, Co, X, Y, Z))
    dx, dw = backward3d(x, w, g, m1, m2, m3)
    rx, rw = torch_grads(x, w, g, (m1, m2, m3))
    ex, ew = _rel(dx, rx), _rel(dw, rw)
    return ex <= 1e-12 and ew <= 1e-12, f"3D torch autograd: dx {ex:.2e} dw {ew:.2e}"


def check_backward3d_adjoint(backward3d, rng):
    B, Ci, Co, X, Y, Z, m1, m2, m3 = 1, 2, 2, 8, 16, 8, 3, 2, 3
    x = rng.standard_normal((B, Ci, X, Y, Z))
    w = _cplx(rng, (2 * m1, 2 * m2, m3, Ci, Co))
    g = rng.standard_normal((B, Co, X, Y, Z))
    dx, dw = backward3d(x, w, g, m1, m2, m3)
    v = rng.standard_normal(x.shape)
    u = _cplx(rng, w.shape)
    lhs_x = float((g * numpy_layer3d(v, w, m1, m2, m3)).sum())
    lhs_w = float((g * numpy_layer3d(x, u, m1, m2, m3)).sum())
    ex = abs(lhs_x - float((dx * v).sum())) / abs(lhs_x)
    ew = abs(lhs_w - float(np.real(np.conj(dw) * u).sum())) / abs(lhs_w)
    return ex <= 1e-11 and ew <= 1e-11, f"3D adjoint identity: x {ex:.2e} w {ew:.2e}"


PINS_2D_BACKWARD = [check_backward2d_torch, check_backward2d_adjoint, check_backward2d_closed_forms]
PINS_3D_BACKWARD = [check_backward3d_torch, check_backward3d_adjoint]
