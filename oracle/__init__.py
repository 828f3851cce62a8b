"""f64 CPU oracle for the selective-scan hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the package smoke check and the CPU-baseline leg of the benchmark
may import this package.  The product (the HIP library and its binding) never does.

Thin ctypes wrapper over ``liboracle.so`` (built from ``oracle.c`` by ``build.py``).
Every function takes numpy arrays, converts them to contiguous float64 and returns
freshly allocated float64 outputs.  What each routine computes, and which page and
section it follows, is stated in ``oracle.c``.

Parity status: every function here is pinned by the CPU tests (closed forms, finite
differences, the unrolled form, step/split equivalence, invariants, page formulas and
hand-derived worked examples under ``tests/golden``).  One exception: the sigmoid-gated
scan (alpha_scan_fwd/bwd) is "parity unpinned" against the pages -- they name the
operation without printing its recurrence, so its forward is a stated reading; that
reading's implementation is pinned (closed forms, the unrolled form, limits) and its
backward is pinned to its forward by central differences and exact identities.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.c_int64


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        sigs = {
            "oracle_scan_fwd": [_I] * 4 + [_D] * 9,
            "oracle_scan_step": [_I] * 3 + [_D] * 8,
            "oracle_scan_materialized": [_I] * 4 + [_D] * 8,
            "oracle_scan_bwd": [_I] * 4 + [_D] * 15,
            "oracle_conv1d_fwd": [_I] * 4 + [_D] * 4,
            "oracle_conv1d_step": [_I] * 3 + [_D] * 5,
            "oracle_conv1d_bwd": [_I] * 4 + [_D] * 6,
            "oracle_conv1d_step_bwd": [_I] * 2 + [_D] * 6,
            "oracle_rmsnorm_fwd": [_I] * 2 + [_D, _D, ctypes.c_double, _D, _D],
            "oracle_rmsnorm_bwd": [_I] * 2 + [_D] * 6,
            "oracle_sigmoid": [_I] + [_D] * 2,
            "oracle_silu": [_I] + [_D] * 2,
            "oracle_silu_grad": [_I] + [_D] * 3,
            "oracle_softplus": [_I] + [_D] * 2,
            "oracle_alpha_scan_fwd": [_I] * 4 + [_D] * 6,
            "oracle_alpha_scan_bwd": [_I] * 4 + [_D] * 8,
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return ctypes.cast(None, _D)
    return a.ctypes.data_as(_D)


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all host cores)."""
    return int(_load().oracle_num_threads())


# ----------------------------------------------------------------------------------
# selective scan
# ----------------------------------------------------------------------------------

def scan_fwd(x, delta, A, Bm, Cm, Dv, h0=None):
    """Returns (y [B,L,D], h_last [B,D,N])."""
    x, delta, A, Bm, Cm, Dv, h0 = map(_f64, (x, delta, A, Bm, Cm, Dv, h0))
    Bsz, L, D = x.shape
    N = A.shape[1]
    y = np.empty((Bsz, L, D))
    h_last = np.empty((Bsz, D, N))
    _load().oracle_scan_fwd(Bsz, L, D, N, _p(x), _p(delta), _p(A), _p(Bm), _p(Cm), _p(Dv),
                            _p(h0), _p(y), _p(h_last))
    return y, h_last


def scan_step(h, x_t, delta_t, A, B_t, C_t, Dv):
    """One token: h [B,D,N] -> (h', y_t [B,D]); x_t, delta_t [B,D]; B_t, C_t [B,N]."""
    h = _f64(h).copy()
    x_t, delta_t, A, B_t, C_t, Dv = map(_f64, (x_t, delta_t, A, B_t, C_t, Dv))
    Bsz, D, N = h.shape
    y = np.empty((Bsz, D))
    _load().oracle_scan_step(Bsz, D, N, _p(h), _p(x_t), _p(delta_t), _p(A), _p(B_t), _p(C_t),
                             _p(Dv), _p(y))
    return h, y


def scan_materialized(x, delta, A, Bm, Cm, Dv, h0=None):
    """O(L^2) unrolled form of the scan output y [B,L,D]."""
    x, delta, A, Bm, Cm, Dv, h0 = map(_f64, (x, delta, A, Bm, Cm, Dv, h0))
    Bsz, L, D = x.shape
    N = A.shape[1]
    y = np.empty((Bsz, L, D))
    _load().oracle_scan_materialized(Bsz, L, D, N, _p(x), _p(delta), _p(A), _p(Bm), _p(Cm),
                                     _p(Dv), _p(h0), _p(y))
    return y


def scan_bwd(x, delta, A, Bm, Cm, Dv, dy, h0=None):
    """Exact adjoint.  Returns dict dx, ddelta, dA, dB, dC, dD, dh0 (dA, dD from zero)."""
    x, delta, A, Bm, Cm, Dv, dy, h0 = map(_f64, (x, delta, A, Bm, Cm, Dv, dy, h0))
    Bsz, L, D = x.shape
    N = A.shape[1]
    out = dict(dx=np.empty((Bsz, L, D)), ddelta=np.empty((Bsz, L, D)), dA=np.zeros((D, N)),
               dB=np.empty((Bsz, L, N)), dC=np.empty((Bsz, L, N)), dD=np.zeros(D),
               dh0=np.empty((Bsz, D, N)))
    _load().oracle_scan_bwd(Bsz, L, D, N, _p(x), _p(delta), _p(A), _p(Bm), _p(Cm), _p(Dv),
                            _p(h0), _p(dy), _p(out["dx"]), _p(out["ddelta"]), _p(out["dA"]),
                            _p(out["dB"]), _p(out["dC"]), _p(out["dD"]), _p(out["dh0"]))
    return out


# ----------------------------------------------------------------------------------
# conv1d
# ----------------------------------------------------------------------------------

def conv1d_step(state, x_t, W, bias=None):
    """One token: state [B,K-1,D] (last K-1 inputs, oldest first) -> (state', out_t [B,D])."""
    state = _f64(state).copy()
    x_t, W, bias = map(_f64, (x_t, W, bias))
    Bsz, D = x_t.shape
    K = W.shape[1]
    out = np.empty((Bsz, D))
    _load().oracle_conv1d_step(Bsz, D, K, _p(state), _p(x_t), _p(W), _p(bias), _p(out))
    return state, out


def conv1d_fwd(x, W, bias=None):
    x, W, bias = map(_f64, (x, W, bias))
    Bsz, L, D = x.shape
    K = W.shape[1]
    out = np.empty((Bsz, L, D))
    _load().oracle_conv1d_fwd(Bsz, L, D, K, _p(x), _p(W), _p(bias), _p(out))
    return out


def conv1d_bwd(x, W, dout):
    """Returns dict dx [B,L,D], dW [D,K], db [D] (dW, db from zero)."""
    x, W, dout = map(_f64, (x, W, dout))
    Bsz, L, D = x.shape
    K = W.shape[1]
    out = dict(dx=np.empty((Bsz, L, D)), dW=np.zeros((D, K)), db=np.zeros(D))
    _load().oracle_conv1d_bwd(Bsz, L, D, K, _p(x), _p(W), _p(dout), _p(out["dx"]),
                              _p(out["dW"]), _p(out["db"]))
    return out


def conv1d_step_bwd(d_out, window, W, dW=None, db=None):
    """The per-timestep step backward; dW, db are accumulated (copies returned)."""
    d_out, window, W = map(_f64, (d_out, window, W))
    D, K = W.shape
    dW = np.zeros((D, K)) if dW is None else _f64(dW).copy()
    db = np.zeros(D) if db is None else _f64(db).copy()
    dx = np.empty(D)
    _load().oracle_conv1d_step_bwd(D, K, _p(d_out), _p(window), _p(W), _p(dx), _p(dW), _p(db))
    return dx, dW, db


# ----------------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------------

def rmsnorm_fwd(x, scale, eps):
    x, scale = map(_f64, (x, scale))
    R, M = x.shape
    y = np.empty((R, M))
    rms = np.empty(R)
    _load().oracle_rmsnorm_fwd(R, M, _p(x), _p(scale), float(eps), _p(y), _p(rms))
    return y, rms


def rmsnorm_residual_fwd(x, residual, scale, eps):
    """The norm with the residual stream added first (the Mamba block's add-then-norm):
    h = x + residual, then rmsnorm_fwd(h).  Returns (y, rms, h); h is the residual stream
    passed on, and the backward of the norm takes it as its input."""
    h = _f64(x) + _f64(residual)
    y, rms = rmsnorm_fwd(h, scale, eps)
    return y, rms, h


def rmsnorm_bwd(dy, x, scale, rms):
    """Returns dict dx [R,M], dscale [M] (dscale from zero)."""
    dy, x, scale, rms = map(_f64, (dy, x, scale, rms))
    R, M = x.shape
    out = dict(dx=np.empty((R, M)), dscale=np.zeros(M))
    _load().oracle_rmsnorm_bwd(R, M, _p(dy), _p(x), _p(scale), _p(rms), _p(out["dx"]),
                               _p(out["dscale"]))
    return out


# ----------------------------------------------------------------------------------
# elementwise neighbours of the scan
# ----------------------------------------------------------------------------------

def _elementwise(name, *arrays):
    arrays = [np.ascontiguousarray(_f64(a)) for a in arrays]
    out = np.empty_like(arrays[0])
    getattr(_load(), name)(arrays[0].size, *[_p(a) for a in arrays], _p(out))
    return out


def sigmoid(p):
    return _elementwise("oracle_sigmoid", p)


def silu(p):
    return _elementwise("oracle_silu", p)


def silu_grad(p, dout):
    """dout * silu'(p)."""
    return _elementwise("oracle_silu_grad", p, dout)


def softplus(z):
    return _elementwise("oracle_softplus", z)


# ----------------------------------------------------------------------------------
# the scan with its neighbours (Mamba block): time-step activation and output gate
# ----------------------------------------------------------------------------------

def _pre_delta(delta_raw, delta_bias):
    pre = _f64(delta_raw)
    if delta_bias is not None:
        pre = pre + _f64(delta_bias)[None, None, :]
    return pre


def scan_fused_fwd(x, delta_raw, A, Bm, Cm, Dv, h0=None, delta_bias=None,
                   delta_softplus=False, z=None):
    """The scan between its neighbours in the Mamba block, step by step:
      1. time step: pre = delta_raw + delta_bias[d];  delta = softplus(pre) when
         delta_softplus, else pre (dt_proj's output and bias, made positive);
      2. the selective scan with that delta (scan_fwd);
      3. output gate: out = y * silu(z) when z is given, else out = y.
    Returns dict out, y (before the gate), h_last, delta (the scan's time step)."""
    pre = _pre_delta(delta_raw, delta_bias)
    delta = softplus(pre) if delta_softplus else pre
    y, h_last = scan_fwd(x, delta, A, Bm, Cm, Dv, h0)
    out = y * silu(z) if z is not None else y
    return dict(out=out, y=y, h_last=h_last, delta=delta)


def scan_fused_bwd(x, delta_raw, A, Bm, Cm, Dv, dout, h0=None, delta_bias=None,
                   delta_softplus=False, z=None):
    """Gradients of scan_fused_fwd's out for upstream dout, by the chain rule through its
    three steps in reverse:
      3. gate:  dy = dout * silu(z),  dz = (dout * y) * silu'(z)   (y recomputed);
      2. scan:  scan_bwd with dy, giving the gradient d(delta) of the scan's time step;
      1. time step: ddelta = d(delta) * sigmoid(pre) when delta_softplus (softplus' is
         the sigmoid), else d(delta); d(delta_bias)[d] = sum over batch and time of it.
    Returns dict dx, ddelta (with respect to delta_raw), dA, dB, dC, dD, dh0, dz (None
    without z), ddelta_bias."""
    pre = _pre_delta(delta_raw, delta_bias)
    delta = softplus(pre) if delta_softplus else pre
    dout = _f64(dout)
    dz = None
    if z is not None:
        y, _ = scan_fwd(x, delta, A, Bm, Cm, Dv, h0)
        dy = dout * silu(z)
        dz = silu_grad(z, dout * y)
    else:
        dy = dout
    r = scan_bwd(x, delta, A, Bm, Cm, Dv, dy, h0)
    if delta_softplus:
        r["ddelta"] = r["ddelta"] * sigmoid(pre)
    r["ddelta_bias"] = r["ddelta"].sum(axis=(0, 1))
    r["dz"] = dz
    return r


def scan_fused_step(h, x_t, delta_t, A, B_t, C_t, Dv, delta_bias=None, delta_softplus=False,
                    z_t=None):
    """One token of scan_fused_fwd: the time step softplus(delta_t + delta_bias) (or
    without the softplus), one scan step, then the gate y_t * silu(z_t).  Returns
    (h', out_t)."""
    pre = _f64(delta_t)
    if delta_bias is not None:
        pre = pre + _f64(delta_bias)[None, :]
    dt = softplus(pre) if delta_softplus else pre
    h2, y = scan_step(h, x_t, dt, A, B_t, C_t, Dv)
    return h2, (y * silu(z_t) if z_t is not None else y)


def decode_step(h, conv_state, x_t, W, conv_bias, delta_t, A, B_t, C_t, Dv, delta_bias=None,
                delta_softplus=False, z_t=None):
    """One token of the Mamba block's scan branch: the conv step on x_t, its SiLU, then the
    fused scan step on that input.  Returns (h', conv_state', out_t)."""
    state2, c = conv1d_step(conv_state, x_t, W, conv_bias)
    h2, out = scan_fused_step(h, silu(c), delta_t, A, B_t, C_t, Dv, delta_bias=delta_bias,
                              delta_softplus=delta_softplus, z_t=z_t)
    return h2, state2, out


# ----------------------------------------------------------------------------------
# sigmoid-gated scan (foxhunt ml-alpha forward-pass commit; parity unpinned, see oracle.c)
# ----------------------------------------------------------------------------------

def alpha_scan_fwd(a, b, Wc, h0=None):
    """a, b [Bn,K,S]; Wc [H,S]; h0 [Bn,H] or None.  Returns (h [Bn,H], x_last [Bn,S])."""
    a, b, Wc, h0 = map(_f64, (a, b, Wc, h0))
    Bn, K, S = a.shape
    H = Wc.shape[0]
    h = np.empty((Bn, H))
    xl = np.empty((Bn, S))
    _load().oracle_alpha_scan_fwd(Bn, K, S, H, _p(a), _p(b), _p(Wc), _p(h0), _p(h), _p(xl))
    return h, xl


def alpha_scan_bwd(a, b, Wc, dh):
    """Exact adjoint for upstream gradient dh [Bn,H].  Returns dict da, db, dWc (from
    zero), dh0."""
    a, b, Wc, dh = map(_f64, (a, b, Wc, dh))
    Bn, K, S = a.shape
    H = Wc.shape[0]
    out = dict(da=np.empty((Bn, K, S)), db=np.empty((Bn, K, S)), dWc=np.zeros((H, S)),
               dh0=np.empty((Bn, H)))
    _load().oracle_alpha_scan_bwd(Bn, K, S, H, _p(a), _p(b), _p(Wc), _p(dh), _p(out["da"]),
                                  _p(out["db"]), _p(out["dWc"]), _p(out["dh0"]))
    return out
