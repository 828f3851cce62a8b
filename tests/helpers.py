"""Shared test helpers: error metrics and central finite differences (test code)."""
import numpy as np


def rel_err(got, ref):
    """Normwise max relative error: max|got - ref| / max|ref| (0 if both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def fd_grad(fun, theta, step_rel=1e-5):
    """Central differences of the scalar fun at theta (any shape), f64."""
    theta = np.array(theta, dtype=np.float64, copy=True)
    g = np.zeros_like(theta)
    flat = theta.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        h = step_rel * max(1.0, abs(flat[i]))
        old = flat[i]
        flat[i] = old + h
        fp = fun(theta)
        flat[i] = old - h
        fm = fun(theta)
        flat[i] = old
        gf[i] = (fp - fm) / (2.0 * h)
    return g
