"""The float64 oracle against results that mathematics fixes (brute force,
closed forms, invariants, numpy.fft cross-checks), and mutation tests showing
that plausible mistakes in an oracle-like implementation fail those pins.

The pages print no worked example values for the layer, so no pin comes from
them; see tests/golden/README.md.
"""

import numpy as np
import pytest

import oracle
from oracle import spectral as osp
import pins


@pytest.fixture
def rng():
    return np.random.default_rng(pins.RNG_SEED)


@pytest.mark.parametrize("check", pins.PINS_2D_FORWARD, ids=lambda f: f.__name__)
def test_forward2d_pins(check, rng):
    ok, msg = check(oracle.forward2d, rng)
    assert ok, msg


def test_contract_pins(rng):
    ok, msg = pins.check_contract_loops(oracle.contract, rng)
    assert ok, msg


@pytest.mark.parametrize("check", pins.PINS_2D_LAYER, ids=lambda f: f.__name__)
def test_layer2d_pins(check, rng):
    ok, msg = check(oracle.spectral_conv2d, rng)
    assert ok, msg


@pytest.mark.parametrize("check", [pins.check_forward3d_brute, pins.check_forward3d_numpy_delta],
                         ids=lambda f: f.__name__)
def test_forward3d_pins(check, rng):
    ok, msg = check(oracle.forward3d, rng)
    assert ok, msg


@pytest.mark.parametrize("check", [pins.check_layer3d_numpy_pipeline, pins.check_layer3d_identity],
                         ids=lambda f: f.__name__)
def test_layer3d_pins(check, rng):
    ok, msg = check(oracle.spectral_conv3d, rng)
    assert ok, msg


# ------------------------------------------------------------ mutation tests
# Each mutant is the oracle with one plausible mistake planted (on the CPU).
# At least one pin of the relevant group must fail for it.

def _fwd_wrong_sign(x, m1, m2):
    return np.conj(oracle.forward2d(x, m1, m2))


def _fwd_high_corner_offset(x, m1, m2):
    H, W = x.shape[-2:]
    xs = np.roll(x, 1, axis=-2)  # equivalent to a kx-dependent phase error
    out = oracle.forward2d(x, m1, m2)
    out[..., m1:, :] = oracle.forward2d(xs, m1, m2)[..., m1:, :]
    return out


def _fwd_dropped_high_corner(x, m1, m2):
    out = oracle.forward2d(x, m1, m2)
    out[..., m1:, :] = 0
    return out


def _fwd_transposed_axes(x, m1, m2):
    return oracle.forward2d(np.swapaxes(x, -1, -2), m1, m2) if x.shape[-1] == x.shape[-2] \
        else oracle.forward2d(x, m1, m2)[..., ::-1, :]


def _contract_transposed(xh, w):
    return osp.contract(xh, np.swapaxes(w, -1, -2)) if w.shape[-1] == w.shape[-2] \
        else osp.contract(xh, np.conj(w))


def _contract_conjugated(xh, w):
    return osp.contract(xh, np.conj(w))


def _layer_gamma0_doubled(x, w, m1, m2):
    H, W = x.shape[-2:]
    yh = osp.contract(osp.forward2d(x, m1, m2), w)
    y = osp.inverse2d(yh, H, W, m1, m2)
    y0 = osp.inverse2d(np.concatenate([yh[..., :1], 0 * yh[..., 1:]], axis=-1), H, W, m1, m2)
    return y + y0  # ky = 0 term counted twice


def _layer_no_norm(x, w, m1, m2):
    H, W = x.shape[-2:]
    return osp.spectral_conv2d(x, w, m1, m2) * (H * W) / max(H, W)


def _layer_keeps_imag_dc(x, w, m1, m2):
    # c2r mistake: treats the ky = 0 column as if it were complex-symmetric,
    # adding the imaginary part's contribution instead of dropping it
    H, W = x.shape[-2:]
    yh = osp.contract(osp.forward2d(x, m1, m2), w)
    hh = np.arange(H)
    kx = osp.corner_indices(H, m1)
    Z0 = np.einsum("ah,...a->...h", np.exp(2j * np.pi * np.outer(kx, hh) / H), yh[..., 0])
    return osp.inverse2d(yh, H, W, m1, m2) + (Z0.imag / (H * W))[..., :, None]


def _layer_low_corner_only(x, w, m1, m2):
    H, W = x.shape[-2:]
    yh = osp.contract(osp.forward2d(x, m1, m2), w)
    yh[..., m1:, :] = 0
    return osp.inverse2d(yh, H, W, m1, m2)


FWD_MUTANTS = [_fwd_wrong_sign, _fwd_high_corner_offset, _fwd_dropped_high_corner,
               _fwd_transposed_axes]
LAYER_MUTANTS = [_layer_gamma0_doubled, _layer_no_norm, _layer_keeps_imag_dc,
                 _layer_low_corner_only]


@pytest.mark.parametrize("mutant", FWD_MUTANTS, ids=lambda f: f.__name__)
def test_forward_mutants_are_caught(mutant):
    failures = 0
    for check in pins.PINS_2D_FORWARD:
        ok, _ = check(mutant, np.random.default_rng(pins.RNG_SEED))
        failures += (not ok)
    assert failures >= 1


@pytest.mark.parametrize("mutant", [_contract_transposed, _contract_conjugated],
                         ids=lambda f: f.__name__)
def test_contract_mutants_are_caught(mutant):
    ok, _ = pins.check_contract_loops(mutant, np.random.default_rng(pins.RNG_SEED))
    assert not ok


@pytest.mark.parametrize("mutant", LAYER_MUTANTS, ids=lambda f: f.__name__)
def test_layer_mutants_are_caught(mutant):
    failures = 0
    for check in pins.PINS_2D_LAYER:
        ok, _ = check(mutant, np.random.default_rng(pins.RNG_SEED))
        failures += (not ok)
    assert failures >= 1
