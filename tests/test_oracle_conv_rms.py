"""CPU pins of the conv1d and RMSNorm oracles.

Conv1d: the per-timestep step backward of the mamba-rs backward_conv1d_step section,
summed over the sequence with the saved window, must give the sequence-level weight
and bias gradients; its newest-tap input gradient is the full input gradient when
K = 1; central differences of the forward pin every gradient; a per-channel bilinear
identity ties dx, dW and the output together.

RMSNorm: central differences of the textbook forward pin the backward of the mamba-rs
backward_rms_norm section; two exact invariants (scale invariance of the normalised
row at eps = 0, and linearity in the scale) and a worked example complete the pins.
"""
import json
import os

import numpy as np
import pytest

import oracle
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import BY_NAME, custom
from tests.helpers import fd_grad, rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "conv_rms_worked_example.json")


def _conv(w, seed=0):
    t = synth.conv_inputs(w, seed)
    return {k: synth.as_f64(v) for k, v in t.items()}


def _rms(w, seed=0):
    t = synth.rms_inputs(w, seed)
    q = {k: synth.as_f64(v) for k, v in t.items()}
    _, q["rms"] = oracle.rmsnorm_fwd(q["x"], q["scale"], synth.RMS_EPS)  # the saved statistic
    return q


# ---------------------------------------------------------------------------------
# conv1d
# ---------------------------------------------------------------------------------

def test_conv_worked_example():
    g = json.load(open(GOLDEN))["conv"]
    B, L, D, K = g["B"], g["L"], g["D"], g["K"]
    x = np.array(g["x"], dtype=np.float64).reshape(B, L, D)
    W = np.array(g["W"], dtype=np.float64)
    bias = np.array(g["bias"], dtype=np.float64)
    dout = np.array(g["dout"], dtype=np.float64).reshape(B, L, D)
    out = oracle.conv1d_fwd(x, W, bias)
    np.testing.assert_allclose(out.reshape(-1), g["out"], atol=1e-15)
    r = oracle.conv1d_bwd(x, W, dout)
    np.testing.assert_allclose(r["dx"].reshape(-1), g["dx"], atol=1e-15)
    np.testing.assert_allclose(r["dW"], g["dW"], atol=1e-15)
    np.testing.assert_allclose(r["db"], g["db"], atol=1e-15)


def _window(x, b, t, K):
    """Saved shift-register state at time t: window[d, k] = x[b, t-K+1+k, d] (0 before start)."""
    L, D = x.shape[1], x.shape[2]
    win = np.zeros((D, K))
    for k in range(K):
        s = t - K + 1 + k
        if 0 <= s < L:
            win[:, k] = x[b, s]
    return win


@pytest.mark.parametrize("K", [1, 2, 4, 7])
def test_conv_sequence_grads_equal_summed_page_steps(K):
    w = custom(B=2, L=11, D=6, K=K)
    p = _conv(w)
    r = oracle.conv1d_bwd(p["x"], p["W"], p["dout"])
    dW = np.zeros((w.D, K))
    db = np.zeros(w.D)
    for b in range(w.B):
        for t in range(w.L):
            dx_step, dW, db = oracle.conv1d_step_bwd(p["dout"][b, t], _window(p["x"], b, t, K),
                                                     p["W"], dW, db)
            # the newest-tap term is exactly the contribution of output t to dx[b, t]
            np.testing.assert_allclose(dx_step, p["dout"][b, t] * p["W"][:, K - 1], rtol=1e-15)
            if K == 1:
                np.testing.assert_allclose(r["dx"][b, t], dx_step, rtol=1e-15)
    assert rel_err(r["dW"], dW) < 1e-14
    assert rel_err(r["db"], db) < 1e-14


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_conv_step_sequence_equals_full_conv(K):
    # the decode step, started from an all-zero window and fed the sequence one token at
    # a time, gives the full causal conv's output at every step, and ends holding the
    # last K-1 inputs
    w = custom(B=2, L=13, D=5, K=K)
    p = _conv(w)
    bias = synth.as_f64(synth.conv_bias(w))
    full = oracle.conv1d_fwd(p["x"], p["W"], bias)
    state = np.zeros((w.B, K - 1, w.D))
    for t in range(w.L):
        state, o = oracle.conv1d_step(state, p["x"][:, t], p["W"], bias)
        np.testing.assert_allclose(o, full[:, t], rtol=0, atol=1e-13)
    np.testing.assert_array_equal(state, p["x"][:, w.L - (K - 1):, :])


def test_conv_last_step_input_grad_is_newest_tap():
    # at t = L-1 no later output reads x[L-1] through an older tap
    w = custom(B=2, L=9, D=5, K=4)
    p = _conv(w)
    r = oracle.conv1d_bwd(p["x"], p["W"], p["dout"])
    np.testing.assert_allclose(r["dx"][:, -1], p["dout"][:, -1] * p["W"][None, :, -1], rtol=1e-14)


@pytest.mark.parametrize("K", [1, 4])
def test_conv_bwd_matches_central_differences(K):
    w = BY_NAME["tiny"] if K == 4 else custom(B=2, L=8, D=8, K=1)
    p = _conv(w)
    bias = np.linspace(-0.3, 0.4, w.D)
    dout = p["dout"]
    r = oracle.conv1d_bwd(p["x"], p["W"], dout)

    def loss_x(x):
        return float(np.sum(dout * oracle.conv1d_fwd(x, p["W"], bias)))

    def loss_w(Wc):
        return float(np.sum(dout * oracle.conv1d_fwd(p["x"], Wc, bias)))

    def loss_b(bb):
        return float(np.sum(dout * oracle.conv1d_fwd(p["x"], p["W"], bb)))
    assert rel_err(r["dx"], fd_grad(loss_x, p["x"])) < 1e-6
    assert rel_err(r["dW"], fd_grad(loss_w, p["W"])) < 1e-6
    assert rel_err(r["db"], fd_grad(loss_b, bias)) < 1e-6


def test_conv_bilinear_invariant():
    # per channel: sum_{b,t} x dx = sum_k W dW = sum_{b,t} dout (out - bias)
    w = custom(B=3, L=40, D=9, K=4)
    p = _conv(w)
    r = oracle.conv1d_bwd(p["x"], p["W"], p["dout"])
    out = oracle.conv1d_fwd(p["x"], p["W"])
    a = np.einsum("btd,btd->d", p["x"], r["dx"])
    b = np.einsum("dk,dk->d", p["W"], r["dW"])
    c = np.einsum("btd,btd->d", p["dout"], out)
    assert rel_err(a, c) < 1e-13
    assert rel_err(b, c) < 1e-13


def test_conv_accumulates_into_weight_grads():
    w = custom(B=2, L=7, D=4, K=3)
    p = _conv(w)
    dW0 = np.full((4, 3), 0.25)
    db0 = np.full(4, -1.0)
    _, dW1, db1 = oracle.conv1d_step_bwd(p["dout"][0, 3], _window(p["x"], 0, 3, 3), p["W"], dW0, db0)
    np.testing.assert_allclose(db1 - db0, p["dout"][0, 3], rtol=1e-15)
    np.testing.assert_allclose(dW1 - dW0, p["dout"][0, 3][:, None] * _window(p["x"], 0, 3, 3),
                               rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------------

def test_rms_worked_example():
    g = json.load(open(GOLDEN))["rms"]
    x = np.array(g["x"], dtype=np.float64)
    scale = np.array(g["scale"], dtype=np.float64)
    dy = np.array(g["dy"], dtype=np.float64)
    y, rms = oracle.rmsnorm_fwd(x, scale, g["eps"])
    np.testing.assert_allclose(rms, g["rms"], rtol=1e-15)
    np.testing.assert_allclose(y, g["y"], rtol=1e-15)
    r = oracle.rmsnorm_bwd(dy, x, scale, rms)
    np.testing.assert_allclose(r["dx"], g["dx"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["dscale"], g["dscale"], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("eps", [1e-5, 0.3])
def test_rms_bwd_matches_central_differences(eps):
    R, M = 16, 8  # the tiny workload's norm shape (rows = B*L)
    p = _rms(BY_NAME["tiny"])
    x, dy, scale = p["x"], p["dy"], p["scale"]
    assert x.shape == (R, M)
    _, rms = oracle.rmsnorm_fwd(x, scale, eps)
    r = oracle.rmsnorm_bwd(dy, x, scale, rms)

    def loss_x(xx):
        y, _ = oracle.rmsnorm_fwd(xx, scale, eps)
        return float(np.sum(dy * y))

    def loss_s(ss):
        y, _ = oracle.rmsnorm_fwd(x, ss, eps)
        return float(np.sum(dy * y))
    assert rel_err(r["dx"], fd_grad(loss_x, x)) < 1e-6
    assert rel_err(r["dscale"], fd_grad(loss_s, scale)) < 1e-6


def test_rms_invariants():
    w = custom(B=4, L=16, D=24)
    p = _rms(w)
    x, dy, scale = p["x"], p["dy"], p["scale"]
    # eps = 0: y is invariant to scaling a row, so each row's dx is orthogonal to x
    y0, rms0 = oracle.rmsnorm_fwd(x, scale, 0.0)
    r0 = oracle.rmsnorm_bwd(dy, x, scale, rms0)
    rowdot = np.einsum("ri,ri->r", x, r0["dx"])
    assert np.max(np.abs(rowdot)) < 1e-12 * np.max(np.abs(r0["dx"])) * x.shape[1]
    # y is linear in scale: sum_i scale_i dscale_i = sum dy y (any eps)
    y, rms = oracle.rmsnorm_fwd(x, scale, 1e-5)
    r = oracle.rmsnorm_bwd(dy, x, scale, rms)
    assert abs(np.dot(scale, r["dscale"]) - np.sum(dy * y)) < 1e-12 * np.sum(np.abs(dy * y))




# ---------------------------------------------------------------------------------
# the norm with the residual stream added first
# ---------------------------------------------------------------------------------

def test_rms_residual_reduces_to_the_plain_norm_and_is_symmetric():
    w = custom(B=2, L=9, D=40)
    p = _rms(w)
    res = synth.as_f64(synth.rms_residual(w))
    y0, rms0 = oracle.rmsnorm_fwd(p["x"], p["scale"], synth.RMS_EPS)
    y, rms, h = oracle.rmsnorm_residual_fwd(p["x"], np.zeros_like(res), p["scale"], synth.RMS_EPS)
    assert np.array_equal(y, y0) and np.array_equal(rms, rms0) and np.array_equal(h, p["x"])
    a = oracle.rmsnorm_residual_fwd(p["x"], res, p["scale"], synth.RMS_EPS)
    b = oracle.rmsnorm_residual_fwd(res, p["x"], p["scale"], synth.RMS_EPS)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_rms_residual_gradients_are_the_norm_backward_of_the_sum():
    # d/dx and d/dresidual of sum(dy * y(x + residual)) are both the norm's dx at the sum
    w = custom(B=2, L=4, D=6)
    p = _rms(w)
    res = synth.as_f64(synth.rms_residual(w))
    x, dy, scale = p["x"], p["dy"], p["scale"]
    _, rms, h = oracle.rmsnorm_residual_fwd(x, res, scale, synth.RMS_EPS)
    dx = oracle.rmsnorm_bwd(dy, h, scale, rms)["dx"]
    fx = fd_grad(lambda t: float(np.sum(dy * oracle.rmsnorm_residual_fwd(t, res, scale, synth.RMS_EPS)[0])), x)
    fr = fd_grad(lambda t: float(np.sum(dy * oracle.rmsnorm_residual_fwd(x, t, scale, synth.RMS_EPS)[0])), res)
    assert rel_err(dx, fx) < 1e-7
    assert rel_err(dx, fr) < 1e-7
