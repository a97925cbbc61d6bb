"""The float64 backward oracle against its pins (PyTorch autograd through the
torch.fft pipeline, adjoint identities against a numpy.fft forward, closed
forms), and planted mistakes in copies of it that those pins must catch."""

import numpy as np
import pytest

from oracle import backward as ob
from oracle import spectral as osp
import pins
import pins_backward as pb


@pytest.fixture
def rng():
    return np.random.default_rng(pins.RNG_SEED)


@pytest.mark.parametrize("check", pb.PINS_2D_BACKWARD, ids=lambda f: f.__name__)
def test_backward2d_pins(check, rng):
    ok, msg = check(ob.spectral_conv2d_backward, rng)
    assert ok, msg


@pytest.mark.parametrize("check", pb.PINS_3D_BACKWARD, ids=lambda f: f.__name__)
def test_backward3d_pins(check, rng):
    ok, msg = check(ob.spectral_conv3d_backward, rng)
    assert ok, msg


# ------------------------------------------------------------ mutation tests

def _bwd_parts(x, w, g, m1, m2, gh_fn=None, gw_fn=None, adj_fn=None, fT_fn=None):
    H, W = x.shape[-2:]
    gh = (gh_fn or ob.adjoint_inverse2d)(g, m1, m2)
    dw = (gw_fn or ob.contract_grad_w)(osp.forward2d(x, m1, m2), gh)
    dx = (fT_fn or ob.adjoint_forward2d)((adj_fn or ob.contract_adjoint_x)(gh, w), H, W, m1, m2)
    return dx, dw


def _mut_grad_w_no_conj(x, w, g, m1, m2):
    return _bwd_parts(x, w, g, m1, m2, gw_fn=lambda xh, gh: ob.contract_grad_w(np.conj(xh), gh))


def _mut_adjoint_no_conj(x, w, g, m1, m2):
    return _bwd_parts(x, w, g, m1, m2,
                      adj_fn=lambda gh, w_: osp.contract(gh, np.swapaxes(w_, -1, -2)))


def _mut_no_gamma(x, w, g, m1, m2):
    H, W = x.shape[-2:]
    return _bwd_parts(x, w, g, m1, m2, gh_fn=lambda g_, a, b: osp.forward2d(g_, a, b) / (H * W))


def _mut_gamma_on_dx(x, w, g, m1, m2):
    # uses the layer's own inverse (c2r weights, 1/N) in place of F^T
    H, W = x.shape[-2:]
    return _bwd_parts(x, w, g, m1, m2, fT_fn=lambda z, h, w_, a, b: osp.inverse2d(z, h, w_, a, b) * (h * w_))


def _mut_no_norm(x, w, g, m1, m2):
    return _bwd_parts(x, w, g, m1, m2,
                      gh_fn=lambda g_, a, b: ob.adjoint_inverse2d(g_, a, b) * g_.shape[-1])


def _mut_grad_w_conj_out(x, w, g, m1, m2):
    dx, dw = ob.spectral_conv2d_backward(x, w, g, m1, m2)
    return dx, np.conj(dw)


def _mut_high_corner_sign(x, w, g, m1, m2):
    # inverse-sign phase for the high kx corner in F^T
    def fT(z, H, W, a, b):
        zz = z.copy()
        zz[..., a:, :] = np.conj(zz[..., a:, :])
        return ob.adjoint_forward2d(zz, H, W, a, b)
    return _bwd_parts(x, w, g, m1, m2, fT_fn=fT)


MUTANTS = [_mut_grad_w_no_conj, _mut_adjoint_no_conj, _mut_no_gamma, _mut_gamma_on_dx, _mut_no_norm,
           _mut_grad_w_conj_out, _mut_high_corner_sign]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_backward_mutants_are_caught(mutant):
    failures = 0
    for check in pb.PINS_2D_BACKWARD:
        ok, _ = check(mutant, np.random.default_rng(pins.RNG_SEED))
        failures += (not ok)
    assert failures >= 1
