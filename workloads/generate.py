"""Seeded input generators (float64 values, then rounded to the storage dtype).

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload):

* layer input x: drawn first. ``uniform`` draws U[-1, 1); ``grf`` draws one
  independent Gaussian random field per (batch, channel) plane.
* GRF: white N(0, 1) noise per plane, shaped in Fourier space by the square
  root of the power spectrum S(k) = (|k|^2 + 49)^-2.5 over integer signed
  wavenumbers, transformed back (real part), then the whole tensor is scaled
  to unit RMS.
* spectral weights: drawn after x; the real block for the whole weight shape,
  then the imaginary block, each (1 / (Ci * Co)) * U[0, 1).
* storage rounding: round-to-nearest-even from float64. fp16 via numpy;
  bf16 computed exactly (float64 -> float32 with round-to-odd, then RNE to
  the top 16 bits), returned as uint16 bit patterns.

The oracle consumes ``storage_to_float64`` of the stored values, i.e. exactly
the numbers the GPU receives.
"""

import math

import numpy as np

from .configs import LayerConfig, ModelConfig

_STORAGE_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}


def _signed_wavenumbers(n: int) -> np.ndarray:
    k = np.arange(n)
    return np.where(k <= n // 2, k, k - n).astype(np.float64)


def gaussian_random_field(rng: np.random.Generator, lead: tuple, grid: tuple,
                          chunk: int = 8) -> np.ndarray:
    """float64 array of shape lead + grid; unit RMS over the whole array."""
    ks = np.meshgrid(*[_signed_wavenumbers(n) for n in grid], indexing="ij")
    k2 = sum(k * k for k in ks)
    amp = (k2 + 49.0) ** (-1.25)  # sqrt of (|k|^2 + 49)^-2.5
    axes = tuple(range(-len(grid), 0))
    n_planes = int(np.prod(lead)) if lead else 1
    out = np.empty((n_planes,) + tuple(grid), dtype=np.float64)
    for s in range(0, n_planes, chunk):
        e = min(n_planes, s + chunk)
        noise = rng.standard_normal((e - s,) + tuple(grid))
        spec = np.fft.fftn(noise, axes=axes) * amp
        out[s:e] = np.fft.ifftn(spec, axes=axes).real
    rms = math.sqrt(float(np.mean(out * out)))
    out /= rms
    return out.reshape(tuple(lead) + tuple(grid))


def _f64_to_f32_round_to_odd(a: np.ndarray) -> np.ndarray:
    f = a.astype(np.float32)
    back = f.astype(np.float64)
    inexact = back != a
    # step toward zero where RNE went away from zero, then force the low bit
    away = inexact & (np.abs(back) > np.abs(a))
    f = np.where(away, np.nextafter(f, np.float32(0)), f)
    bits = f.view(np.uint32).copy()
    bits[inexact] |= np.uint32(1)
    return bits.view(np.float32)


def _f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    f = _f64_to_f32_round_to_odd(np.asarray(a, dtype=np.float64))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(f)
    r = np.where(nan, np.uint64(0x7FC0), r)
    return r.astype(np.uint16)


def bf16_bits_to_float64(b: np.ndarray) -> np.ndarray:
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage array (float32, float16, or uint16 bf16 bits)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float64).astype(np.float16)
    if dtype == "bf16":
        return _f64_to_bf16_bits(a)
    raise ValueError(dtype)


def storage_to_float64(s: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_float64(s)
    return np.asarray(s).astype(np.float64)


def spectral_weights(rng: np.random.Generator, shape: tuple, c_in: int,
                     c_out: int) -> np.ndarray:
    """complex128 weights, re/im = (1/(c_in*c_out)) * U[0, 1)."""
    scale = 1.0 / (c_in * c_out)
    re = rng.random(shape) * scale
    im = rng.random(shape) * scale
    return re + 1j * im


def complex_to_interleaved(w: np.ndarray) -> np.ndarray:
    """complex array -> float64 array with a trailing (re, im) axis."""
    out = np.empty(w.shape + (2,), dtype=np.float64)
    out[..., 0] = w.real
    out[..., 1] = w.imag
    return out


def layer_inputs(cfg: LayerConfig, dtype: str, batch: int = None,
                 seed: int = None):
    """Seeded inputs of one layer workload.

    Returns dict with ``x`` / ``w`` in storage form (w interleaved re/im on a
    trailing axis of 2) and ``x64`` / ``w64`` (float64 / complex128 copies of
    the stored values, what the oracle consumes). ``batch`` and ``seed``
    override the registry values for reduced-size samples.
    """
    b = cfg.batch if batch is None else batch
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    lead = (b, cfg.c_in)
    if cfg.input_kind == "uniform":
        x = rng.uniform(-1.0, 1.0, size=lead + tuple(cfg.grid))
    else:
        x = gaussian_random_field(rng, lead, tuple(cfg.grid))
    w = spectral_weights(rng, cfg.weight_shape(), cfg.c_in, cfg.c_out)
    xs = round_to_storage(x, dtype)
    ws = round_to_storage(complex_to_interleaved(w), dtype)
    x64 = storage_to_float64(xs, dtype)
    w64i = storage_to_float64(ws, dtype)
    w64 = w64i[..., 0] + 1j * w64i[..., 1]
    return {"x": xs, "w": ws, "x64": x64, "w64": w64, "dtype": dtype}


def layer_grad_output(cfg: LayerConfig, dtype: str, batch: int = None,
                      seed: int = None):
    """Seeded dL/dy for the layer's backward pass: drawn like x (uniform or a
    Gaussian random field of the same spectrum) with c_out channels, from its
    own stream (seed + 1000 unless given). Returns ``g`` (storage form) and
    ``g64`` (float64 copy of the stored values)."""
    b = cfg.batch if batch is None else batch
    rng = np.random.default_rng((cfg.seed + 1000) if seed is None else seed)
    lead = (b, cfg.c_out)
    if cfg.input_kind == "uniform":
        g = rng.uniform(-1.0, 1.0, size=lead + tuple(cfg.grid))
    else:
        g = gaussian_random_field(rng, lead, tuple(cfg.grid))
    gs = round_to_storage(g, dtype)
    return {"g": gs, "g64": storage_to_float64(gs, dtype)}


def model_inputs(cfg: ModelConfig, batch: int = None, grid: tuple = None,
                 seed: int = None):
    """Seeded input and random-init parameters of the full FNO2d model.

    Draw order: the input GRF a (1 channel); lift P (width x 3), p (width);
    per layer: spectral weights (re block, im block, shape (2*m1, m2, w, w)),
    1x1 bypass W (width x width), b (width); projection Q1 (hidden x width),
    q1 (hidden), Q2 (out x hidden), q2 (out). Linear / 1x1 weights and biases
    are U(-1/sqrt(fan_in), 1/sqrt(fan_in)). Every tensor is rounded to the
    storage dtype; ``*64`` entries are the float64 values of what is stored.
    Features are [a, gx, gy] with gx = h/(H-1), gy = w/(W-1).
    """
    b = cfg.batch if batch is None else batch
    H, W = cfg.grid if grid is None else grid
    m1, m2 = cfg.modes
    width, hid = cfg.width, cfg.proj_hidden
    dt = cfg.dtype
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    a = gaussian_random_field(rng, (b, 1), (H, W))

    def lin(fan_out, fan_in):
        bound = 1.0 / math.sqrt(fan_in)
        wt = rng.uniform(-bound, bound, size=(fan_out, fan_in))
        bs = rng.uniform(-bound, bound, size=(fan_out,))
        return wt, bs

    P, p = lin(width, cfg.in_channels)
    layers = []
    for _ in range(cfg.n_layers):
        ws = spectral_weights(rng, (2 * m1, m2, width, width), width, width)
        Wl, bl = lin(width, width)
        layers.append((ws, Wl, bl))
    Q1, q1 = lin(hid, width)
    Q2, q2 = lin(cfg.out_channels, hid)

    gx = np.broadcast_to((np.arange(H) / (H - 1))[:, None], (H, W))
    gy = np.broadcast_to((np.arange(W) / (W - 1))[None, :], (H, W))
    feats = np.empty((b, 3, H, W), dtype=np.float64)
    feats[:, 0] = a[:, 0]
    feats[:, 1] = gx
    feats[:, 2] = gy

    def st(v):
        s = round_to_storage(v, dt)
        return s, storage_to_float64(s, dt)

    out = {"dtype": dt, "grid": (H, W), "batch": b}
    out["features"], out["features64"] = st(feats)
    out["P"], out["P64"] = st(P)
    out["p"], out["p64"] = st(p)
    out["layers"], out["layers64"] = [], []
    for ws, Wl, bl in layers:
        wsi, wsi64 = st(complex_to_interleaved(ws))
        Ws, Ws64 = st(Wl)
        bs, bs64 = st(bl)
        out["layers"].append({"spectral": wsi, "W": Ws, "b": bs})
        out["layers64"].append({"spectral": wsi64[..., 0] + 1j * wsi64[..., 1],
                                "W": Ws64, "b": bs64})
    out["Q1"], out["Q164"] = st(Q1)
    out["q1"], out["q164"] = st(q1)
    out["Q2"], out["Q264"] = st(Q2)
    out["q2"], out["q264"] = st(q2)
    return out
