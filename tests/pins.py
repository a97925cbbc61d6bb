"""Pins for the float64 oracle: checks against results fixed by mathematics.

Each check takes the implementation under test as callables, so the same
checks run on the oracle (must pass) and on deliberately broken copies of it
(must fail), which shows that a plausible mistake is caught.

Nothing here calls the oracle's own helpers: brute force is written out as
plain sums over the full phase, the closed forms are derived by hand, and
the library cross-checks use numpy.fft.
"""

import math

import numpy as np

RNG_SEED = 1234


def corners(n, m):
    return list(range(m)) + list(range(n - m, n))


# ----------------------------------------------------------------- 2D forward

def brute_forward2d(x, m1, m2):
    """Non-separable DFT: one sum over all (h, w) per retained mode."""
    H, W = x.shape[-2:]
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    out = np.zeros(x.shape[:-2] + (2 * m1, m2), dtype=np.complex128)
    for a, kx in enumerate(corners(H, m1)):
        for ky in range(m2):
            ph = np.exp(-2j * np.pi * (kx * hh / H + ky * ww / W))
            out[..., a, ky] = (x * ph).sum(axis=(-2, -1))
    return out


def check_forward2d_brute(forward2d, rng):
    for (H, W, m1, m2) in [(16, 16, 4, 4), (8, 16, 3, 5), (16, 8, 8, 4)]:
        x = rng.standard_normal((2, 3, H, W))
        got = forward2d(x, m1, m2)
        ref = brute_forward2d(x, m1, m2)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        if not err <= 1e-13:
            return False, f"brute force {H}x{W}: rel err {err:.3e}"
    return True, ""


def check_forward2d_numpy(forward2d, rng):
    H, W, m1, m2 = 32, 16, 6, 5
    x = rng.standard_normal((2, 2, H, W))
    full = np.fft.rfft2(x)
    ref = full[..., corners(H, m1), :][..., :m2]
    got = forward2d(x, m1, m2)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    return err <= 1e-12, f"numpy rfft2 rel err {err:.3e}"


def check_forward2d_delta_const(forward2d, rng):
    H, W, m1, m2 = 16, 16, 4, 4
    h0, w0 = 3, 11
    x = np.zeros((H, W))
    x[h0, w0] = 1.0
    got = forward2d(x, m1, m2)
    for a, kx in enumerate(corners(H, m1)):
        for ky in range(m2):
            ref = complex(math.cos(2 * math.pi * (kx * h0 / H + ky * w0 / W)),
                          -math.sin(2 * math.pi * (kx * h0 / H + ky * w0 / W)))
            if abs(got[a, ky] - ref) > 1e-14:
                return False, f"delta at ({kx},{ky}): {got[a, ky]} vs {ref}"
    c = 0.75
    got = forward2d(np.full((H, W), c), m1, m2)
    ref = np.zeros_like(got)
    ref[0, 0] = c * H * W
    err = np.abs(got - ref).max()
    return err <= 1e-12, f"constant field err {err:.3e}"


def check_forward2d_cosine(forward2d, rng):
    H, W, m1, m2 = 16, 16, 4, 4
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    for p, q in [(2, 1), (-3, 2), (0, 3), (4, 1), (-4, 2)]:
        x = np.cos(2 * np.pi * (p * hh / H + q * ww / W))
        got = forward2d(x, m1, m2)
        ref = np.zeros_like(got)
        kxs = corners(H, m1)
        if (p % H) in kxs:
            ref[kxs.index(p % H), q] = H * W / 2
        err = np.abs(got - ref).max()
        if not err <= 1e-11:
            return False, f"cosine (p={p}, q={q}) err {err:.3e}"
    return True, ""


def check_forward2d_parseval(forward2d, rng):
    """Band-limited field (no Nyquist content): sum |x|^2 equals
    (1/HW) * (sum_{ky=0} |X|^2 + 2 sum_{ky>=1} |X|^2) over the half spectrum."""
    H, W = 16, 16
    spec = rng.standard_normal((H, W // 2 + 1)) + 1j * rng.standard_normal((H, W // 2 + 1))
    spec[:, W // 2] = 0
    spec[H // 2, :] = 0
    x = np.fft.irfft2(spec, s=(H, W))
    X = forward2d(x, H // 2, W // 2)
    e_sp = (np.abs(X[:, 0]) ** 2).sum() + 2 * (np.abs(X[:, 1:]) ** 2).sum()
    e_x = (x ** 2).sum()
    err = abs(e_sp / (H * W) - e_x) / e_x
    return err <= 1e-12, f"Parseval rel err {err:.3e}"


# --------------------------------------------------------------- contraction

def check_contract_loops(contract, rng):
    B, Ci, Co, ms = 2, 3, 5, (4, 2)
    xh = rng.standard_normal((B, Ci) + ms) + 1j * rng.standard_normal((B, Ci) + ms)
    w = rng.standard_normal(ms + (Ci, Co)) + 1j * rng.standard_normal(ms + (Ci, Co))
    ref = np.zeros((B, Co) + ms, dtype=np.complex128)
    for b in range(B):
        for o in range(Co):
            for a in range(ms[0]):
                for k in range(ms[1]):
                    acc = 0j
                    for i in range(Ci):
                        acc += xh[b, i, a, k] * w[a, k, i, o]
                    ref[b, o, a, k] = acc
    got = contract(xh, w)
    err = np.abs(got - ref).max()
    if not err <= 1e-13:
        return False, f"loop contraction err {err:.3e}"
    # w = a * delta_io gives a * xh
    C = 4
    xh = rng.standard_normal((B, C) + ms) + 1j * rng.standard_normal((B, C) + ms)
    a = 0.3 - 0.7j
    w = np.zeros(ms + (C, C), dtype=np.complex128)
    for i in range(C):
        w[..., i, i] = a
    err = np.abs(contract(xh, w) - a * xh).max()
    return err <= 1e-14, f"delta weights err {err:.3e}"


# ------------------------------------------------------------- whole 2D layer

def identity_weights(mshape, C):
    w = np.zeros(tuple(mshape) + (C, C), dtype=np.complex128)
    for i in range(C):
        w[..., i, i] = 1.0
    return w


def lowpass_mask2d(H, W, m1, m2):
    """Real point-symmetric mask over the full spectrum that the identity
    layer applies: retained corners for ky in [1, m2) and their mirror, and
    on ky = 0 weight 1 for |kx| <= m1 - 1 and 1/2 at kx = +-m1 (the c2r
    convention keeps the real part of the ky = 0 term)."""
    M = np.zeros((H, W))
    for kx in range(H):
        s = kx if kx < H // 2 else kx - H  # signed
        for ky in range(W):
            t = ky if ky <= W // 2 else ky - W
            if 1 <= t <= m2 - 1 and -m1 <= s <= m1 - 1:
                M[kx, ky] = 1.0
            elif -(m2 - 1) <= t <= -1 and -(m1 - 1) <= s <= m1:
                M[kx, ky] = 1.0
            elif t == 0:
                if abs(s) <= m1 - 1:
                    M[kx, ky] = 1.0
                elif abs(s) == m1:
                    M[kx, ky] = 0.5
    return M


def check_layer2d_identity_lowpass(layer2d, rng):
    B, C, H, W, m1, m2 = 2, 3, 16, 16, 4, 4
    x = rng.standard_normal((B, C, H, W))
    y = layer2d(x, identity_weights((2 * m1, m2), C), m1, m2)
    M = lowpass_mask2d(H, W, m1, m2)
    ref = np.fft.ifft2(np.fft.fft2(x) * M).real
    err = np.abs(y - ref).max() / np.abs(ref).max()
    if not err <= 1e-12:
        return False, f"identity low-pass err {err:.3e}"
    # Parseval of the projection: ||y||^2 = (1/HW) sum M^2 |X|^2
    X = np.fft.fft2(x)
    e_ref = (M ** 2 * np.abs(X) ** 2).sum() / (H * W)
    e = (y ** 2).sum()
    rel = abs(e - e_ref) / e_ref
    return rel <= 1e-12, f"identity Parseval rel err {rel:.3e}"


def check_layer2d_numpy_pipeline(layer2d, rng):
    """Random complex weights (non-Hermitian ky = 0 column): equals the
    numpy rfft2 -> per-mode einsum -> irfft2 pipeline."""
    B, Ci, Co, H, W, m1, m2 = 2, 3, 4, 16, 32, 5, 7
    x = rng.standard_normal((B, Ci, H, W))
    w = rng.standard_normal((2 * m1, m2, Ci, Co)) + 1j * rng.standard_normal((2 * m1, m2, Ci, Co))
    X = np.fft.rfft2(x)
    Y = np.zeros((B, Co, H, W // 2 + 1), dtype=np.complex128)
    kx = corners(H, m1)
    Y[:, :, kx, :m2] = np.einsum("biay,ayio->boay", X[:, :, kx, :m2], w)
    ref = np.fft.irfft2(Y, s=(H, W))
    got = layer2d(x, w, m1, m2)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    return err <= 1e-12, f"numpy pipeline rel err {err:.3e}"


def check_layer2d_sinusoids(layer2d, rng):
    H, W, m1, m2 = 16, 16, 4, 4
    hh, ww = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    w = identity_weights((2 * m1, m2), 1)
    cases = [((2, 1), 1.0), ((-4, 3), 1.0), ((3, 3), 1.0), ((4, 1), 0.0),
             ((1, 4), 0.0), ((0, 6), 0.0), ((3, 0), 1.0), ((4, 0), 0.5),
             ((-4, 0), 0.5), ((0, 0), 1.0)]
    for (p, q), factor in cases:
        x = np.cos(2 * np.pi * (p * hh / H + q * ww / W))[None, None]
        y = layer2d(x, w, m1, m2)
        err = np.abs(y - factor * x).max()
        if not err <= 1e-13:
            return False, f"sinusoid (p={p}, q={q}) expected {factor}*x, err {err:.3e}"
    return True, ""


def check_layer2d_invariants(layer2d, rng):
    B, Ci, Co, H, W, m1, m2 = 2, 3, 2, 16, 16, 3, 4
    x = rng.standard_normal((B, Ci, H, W))
    x2 = rng.standard_normal((B, Ci, H, W))
    w = rng.standard_normal((2 * m1, m2, Ci, Co)) + 1j * rng.standard_normal((2 * m1, m2, Ci, Co))
    w2 = rng.standard_normal((2 * m1, m2, Ci, Co)) + 1j * rng.standard_normal((2 * m1, m2, Ci, Co))
    y = layer2d(x, w, m1, m2)
    scale = np.abs(y).max()
    ys = layer2d(np.roll(x, (3, -5), axis=(-2, -1)), w, m1, m2)
    e1 = np.abs(ys - np.roll(y, (3, -5), axis=(-2, -1))).max() / scale
    e2 = np.abs(layer2d(2.0 * x - 0.5 * x2, w, m1, m2)
                - (2.0 * y - 0.5 * layer2d(x2, w, m1, m2))).max() / scale
    e3 = np.abs(layer2d(x, w + 3.0 * w2, m1, m2)
                - (y + 3.0 * layer2d(x, w2, m1, m2))).max() / scale
    ok = e1 <= 1e-12 and e2 <= 1e-12 and e3 <= 1e-12 and np.isrealobj(y)
    return ok, f"shift {e1:.2e} lin-x {e2:.2e} lin-w {e3:.2e}"


# ------------------------------------------------------------------------ 3D

def brute_forward3d(x, m1, m2, m3):
    X, Y, Z = x.shape[-3:]
    gx, gy, gz = np.meshgrid(np.arange(X), np.arange(Y), np.arange(Z), indexing="ij")
    out = np.zeros(x.shape[:-3] + (2 * m1, 2 * m2, m3), dtype=np.complex128)
    for a, kx in enumerate(corners(X, m1)):
        for b, ky in enumerate(corners(Y, m2)):
            for kz in range(m3):
                ph = np.exp(-2j * np.pi * (kx * gx / X + ky * gy / Y + kz * gz / Z))
                out[..., a, b, kz] = (x * ph).sum(axis=(-3, -2, -1))
    return out


def check_forward3d_brute(forward3d, rng):
    for (X, Y, Z, m1, m2, m3) in [(8, 8, 8, 2, 2, 2), (4, 8, 16, 2, 3, 5)]:
        x = rng.standard_normal((2, X, Y, Z))
        got = forward3d(x, m1, m2, m3)
        ref = brute_forward3d(x, m1, m2, m3)
        err = np.abs(got - ref).max() / np.abs(ref).max()
        if not err <= 1e-13:
            return False, f"3D brute force rel err {err:.3e}"
    return True, ""


def check_forward3d_numpy_delta(forward3d, rng):
    X, Y, Z, m1, m2, m3 = 8, 16, 8, 3, 4, 3
    x = rng.standard_normal((2, X, Y, Z))
    full = np.fft.rfftn(x, axes=(-3, -2, -1))
    ref = full[..., corners(X, m1), :, :][..., corners(Y, m2), :][..., :m3]
    got = forward3d(x, m1, m2, m3)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    if not err <= 1e-12:
        return False, f"numpy rfftn rel err {err:.3e}"
    d = np.zeros((X, Y, Z))
    p = (5, 2, 7)
    d[p] = 1.0
    got = forward3d(d, m1, m2, m3)
    for a, kx in enumerate(corners(X, m1)):
        for b, ky in enumerate(corners(Y, m2)):
            for kz in range(m3):
                th = 2 * math.pi * (kx * p[0] / X + ky * p[1] / Y + kz * p[2] / Z)
                if abs(got[a, b, kz] - complex(math.cos(th), -math.sin(th))) > 1e-14:
                    return False, "3D delta closed form"
    return True, ""


def check_layer3d_numpy_pipeline(layer3d, rng):
    B, Ci, Co, X, Y, Z, m1, m2, m3 = 2, 3, 2, 8, 8, 16, 2, 3, 4
    x = rng.standard_normal((B, Ci, X, Y, Z))
    ws = (2 * m1, 2 * m2, m3, Ci, Co)
    w = rng.standard_normal(ws) + 1j * rng.standard_normal(ws)
    F = np.fft.rfftn(x, axes=(-3, -2, -1))
    kx, ky = corners(X, m1), corners(Y, m2)
    sel = F[:, :, kx][:, :, :, ky][..., :m3]
    Yf = np.zeros((B, Co, X, Y, Z // 2 + 1), dtype=np.complex128)
    Yf[np.ix_(range(B), range(Co), kx, ky, range(m3))] = np.einsum("nixyz,xyzio->noxyz", sel, w)
    ref = np.fft.irfftn(Yf, s=(X, Y, Z), axes=(-3, -2, -1))
    got = layer3d(x, w, m1, m2, m3)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    return err <= 1e-12, f"3D numpy pipeline rel err {err:.3e}"


def lowpass_mask3d(X, Y, Z, m1, m2, m3):
    """Identity-weight 3D projection: as in 2D, with corners in kx, ky and the
    half spectrum along kz; on kz = 0 the retained set R and its mirror -R
    each carry weight 1/2."""
    M = np.zeros((X, Y, Z))

    def signed(k, n):
        return k if k < n // 2 else k - n

    for i in range(X):
        for j in range(Y):
            for k in range(Z):
                s, t, u = signed(i, X), signed(j, Y), signed(k, Z)
                inR = (-m1 <= s <= m1 - 1) and (-m2 <= t <= m2 - 1) and (0 <= u <= m3 - 1)
                inRm = (-(m1 - 1) <= s <= m1) and (-(m2 - 1) <= t <= m2) and (-(m3 - 1) <= u <= 0)
                if u == 0:
                    M[i, j, k] = 0.5 * inR + 0.5 * inRm
                else:
                    M[i, j, k] = 1.0 if (inR or inRm) else 0.0
    return M


def check_layer3d_identity(layer3d, rng):
    B, C, X, Y, Z, m1, m2, m3 = 1, 2, 8, 8, 8, 2, 3, 2
    x = rng.standard_normal((B, C, X, Y, Z))
    w = identity_weights((2 * m1, 2 * m2, m3), C)
    y = layer3d(x, w, m1, m2, m3)
    M = lowpass_mask3d(X, Y, Z, m1, m2, m3)
    ref = np.fft.ifftn(np.fft.fftn(x, axes=(-3, -2, -1)) * M, axes=(-3, -2, -1)).real
    err = np.abs(y - ref).max() / np.abs(ref).max()
    if not err <= 1e-12:
        return False, f"3D identity low-pass err {err:.3e}"
    gx, gy, gz = np.meshgrid(np.arange(X), np.arange(Y), np.arange(Z), indexing="ij")
    w1 = identity_weights((2 * m1, 2 * m2, m3), 1)
    for (p, q, r), factor in [((1, 2, 1), 1.0), ((2, -2, 1), 0.0), ((-2, 1, 1), 1.0),
                              ((1, 1, 0), 1.0), ((2, 0, 0), 0.5), ((0, 0, 3), 0.0)]:
        xs = np.cos(2 * np.pi * (p * gx / X + q * gy / Y + r * gz / Z))[None, None]
        e = np.abs(layer3d(xs, w1, m1, m2, m3) - factor * xs).max()
        if not e <= 1e-13:
            return False, f"3D sinusoid ({p},{q},{r}) expected {factor}, err {e:.3e}"
    return True, ""


PINS_2D_FORWARD = [check_forward2d_brute, check_forward2d_numpy,
                   check_forward2d_delta_const, check_forward2d_cosine,
                   check_forward2d_parseval]
PINS_2D_LAYER = [check_layer2d_identity_lowpass, check_layer2d_numpy_pipeline,
                 check_layer2d_sinusoids, check_layer2d_invariants]
