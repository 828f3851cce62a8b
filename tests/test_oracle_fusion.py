"""Pins of the oracle's elementwise neighbours of the scan (SiLU, sigmoid, softplus) and
of the conv + SiLU composition the fused conv kernels are checked against.

Each function is checked against what mathematics fixes independently of its own
formula: closed values, exact identities, and central differences of the function it is
the derivative of.
"""
import numpy as np
import pytest

import oracle
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import custom
from tests.helpers import fd_grad, rel_err

RNG = np.random.default_rng(11)


def test_closed_values():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert oracle.silu_grad(np.array([0.0]), np.array([1.0]))[0] == 0.5
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(oracle.softplus(np.array([0.0]))[0] - np.log(2.0)) < 1e-16
    # far tails: silu(p) -> p and softplus(z) -> z (relative error below one ulp)
    assert abs(oracle.silu(np.array([40.0]))[0] / 40.0 - 1.0) < 1e-15
    assert abs(oracle.softplus(np.array([40.0]))[0] / 40.0 - 1.0) < 1e-15
    assert 0.0 < oracle.softplus(np.array([-40.0]))[0] < 1e-17


def test_exact_identities():
    p = RNG.normal(0.0, 3.0, 200)
    # silu(p) - silu(-p) = p (sigmoid(p) + sigmoid(-p) = 1)
    np.testing.assert_allclose(oracle.silu(p) - oracle.silu(-p), p, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.sigmoid(p) + oracle.sigmoid(-p), 1.0, rtol=0, atol=1e-15)
    # softplus(z) - softplus(-z) = z
    np.testing.assert_allclose(oracle.softplus(p) - oracle.softplus(-p), p, rtol=1e-14, atol=1e-14)


def test_derivatives_match_central_differences():
    p = RNG.normal(0.0, 2.0, 40)
    ones = np.ones_like(p)
    # d silu / dp, elementwise
    fd = np.array([fd_grad(lambda t: float(oracle.silu(t)[0]), np.array([v]))[0] for v in p])
    np.testing.assert_allclose(oracle.silu_grad(p, ones), fd, rtol=1e-7, atol=1e-9)
    # d softplus / dz = sigmoid
    fd = np.array([fd_grad(lambda t: float(oracle.softplus(t)[0]), np.array([v]))[0] for v in p])
    np.testing.assert_allclose(oracle.sigmoid(p), fd, rtol=1e-7, atol=1e-9)


def conv_silu_fwd(x, W, bias):
    return oracle.silu(oracle.conv1d_fwd(x, W, bias))


def conv_silu_bwd(x, W, bias, du):
    """Backward of u = silu(conv(x)) for upstream du: the SiLU backward, then the conv's."""
    g = oracle.silu_grad(oracle.conv1d_fwd(x, W, bias), du)
    return oracle.conv1d_bwd(x, W, g)


@pytest.mark.parametrize("K", [1, 3, 4])
def test_conv_silu_composition_matches_central_differences(K):
    w = custom(B=2, L=6, D=3, K=K)
    c = {k: synth.as_f64(v) for k, v in synth.conv_inputs(w).items()}
    bias = synth.as_f64(synth.conv_bias(w))
    du = c["dout"]
    r = conv_silu_bwd(c["x"], c["W"], bias, du)
    fx = fd_grad(lambda t: float(np.sum(du * conv_silu_fwd(t, c["W"], bias))), c["x"])
    fW = fd_grad(lambda t: float(np.sum(du * conv_silu_fwd(c["x"], t, bias))), c["W"])
    fb = fd_grad(lambda t: float(np.sum(du * conv_silu_fwd(c["x"], c["W"], t))), bias)
    assert rel_err(r["dx"], fx) < 1e-7
    assert rel_err(r["dW"], fW) < 1e-7
    assert rel_err(r["db"], fb) < 1e-7
