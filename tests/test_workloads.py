"""Input generators: determinism, statistics and exact storage rounding."""

import numpy as np

import workloads as wl
from workloads.generate import _f64_to_bf16_bits


def test_registry_minimal_bytes():
    c2 = wl.CONFIGS["c2"]
    assert c2.minimal_bytes("f16") == 570_425_344
    c3 = wl.CONFIGS["c3"]
    assert c3.minimal_bytes("f32") == 402_653_184
    c1 = wl.CONFIGS["c1"]
    assert c1.minimal_bytes("f32") == 71_303_168
    assert c1.minimal_bytes("f16") == 35_651_584
    assert wl.CONFIGS["c0"].minimal_bytes("f32") == 20_480


def test_grf_unit_rms_and_spectrum_decay():
    rng = np.random.default_rng(0)
    f = wl.gaussian_random_field(rng, (2, 3), (64, 64))
    assert f.shape == (2, 3, 64, 64)
    assert abs(np.sqrt(np.mean(f * f)) - 1.0) < 1e-12
    p = np.abs(np.fft.fft2(f)) ** 2
    p = p.mean(axis=(0, 1))
    k = np.fft.fftfreq(64, 1.0 / 64)
    kk = np.sqrt(k[:, None] ** 2 + k[None, :] ** 2)
    low = p[(kk >= 1) & (kk <= 2)].mean()
    high = p[(kk >= 18) & (kk <= 22)].mean()
    # (|k|^2+49)^-2.5 predicts a ratio of about 190 between these rings
    assert 80 < low / high < 400


def test_layer_inputs_deterministic():
    cfg = wl.CONFIGS["c0"]
    a = wl.layer_inputs(cfg, "f32")
    b = wl.layer_inputs(cfg, "f32")
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert a["x"].shape == (2, 4, 16, 16)
    assert a["w"].shape == (8, 4, 4, 4, 2)
    assert a["x"].min() >= -1.0 and a["x"].max() < 1.0
    assert (a["w"] >= 0).all() and (a["w"] < 1.0 / 16).all()


def _bf16_rne_reference(v):
    """Exact RNE by brute force: pick the nearer of the two bf16 neighbours."""
    f32 = np.float32(v)
    bits = np.array([f32]).view(np.uint32)[0]
    base = (int(bits) >> 16) << 16
    cands = []
    for d in (-1, 0, 1, 2):
        b = (base >> 16) + d
        if 0 <= b <= 0xFFFF:
            val = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
            if np.isfinite(val):
                cands.append((abs(float(val) - v), b & 1, b))
    cands.sort()
    best = cands[0]
    ties = [c for c in cands if c[0] == best[0]]
    if len(ties) > 1:
        best = [c for c in ties if c[1] == 0][0]
    return best[2]


def test_bf16_rounding_exact():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(3000), rng.random(1000) * 1e-3,
                           # exact ties and near-ties around bf16 midpoints
                           np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8,
                                     1.0 + 2.0 ** -8 + 2.0 ** -40, -(1.0 + 2.0 ** -8)])])
    got = _f64_to_bf16_bits(vals)
    for v, g in zip(vals, got):
        assert int(g) == _bf16_rne_reference(float(v)), v


def test_storage_roundtrip_f16():
    x = np.array([0.1, -2.5, 1e-6, 65504.0])
    s = wl.round_to_storage(x, "f16")
    assert s.dtype == np.float16
    assert np.array_equal(wl.storage_to_float64(s, "f16"), x.astype(np.float16).astype(np.float64))
