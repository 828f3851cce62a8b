"""Seeded synthetic inputs, shared by the HIP path's tests/benchmark and the oracle.

This module only draws random numbers and rounds them to the storage type; it holds
none of the scan, conv or norm arithmetic.  Everything is generated on the CPU with
one ``torch.Generator`` per tensor, seeded ``seed * 1000 + tensor_id`` in a fixed
tensor order, so the same values can be regenerated without a GPU.

Storage rules:
  * activations (x, delta, B, C, dy, conv x/dout, norm x/dy) are stored in the
    workload's dtype (f32 or bf16, rounded to nearest-even by ``Tensor.to``);
  * parameters (A, D, conv W and bias, norm scale) are f32; for bf16 workloads they
    hold bf16-rounded values, so "cast to bf16" and "f32 parameter" give one number.

The RMSNorm backward also takes the statistic its forward saved (rms); that is the
forward's arithmetic, so it is not drawn here: the tests take it from the oracle's
forward, the benchmark from the library's.
"""
import torch

from .workloads import Workload

# tensor ids (fixed order)
(_X, _DELTA, _B, _C, _DV, _DY, _CX, _CW, _CDOUT, _RX, _RDY, _RSCALE, _H0, _CBIAS, _DRAW, _DBIAS,
 _Z, _RRES, _GA, _GB, _GWC, _GH0, _GDH) = range(1, 24)

RMS_EPS = 1e-5  # the RMSNorm eps of every workload


def _gen(seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + tid)
    return g


def _store_dtype(w: Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _param(t: torch.Tensor, w: Workload) -> torch.Tensor:
    """f32 parameter; bf16-rounded values for bf16 workloads."""
    t = t.to(torch.float32)
    if w.dtype == "bf16":
        t = t.to(torch.bfloat16).to(torch.float32)
    return t.contiguous()


def _normal(shape, seed, tid, mean=0.0, std=1.0):
    return torch.randn(shape, generator=_gen(seed, tid), dtype=torch.float32) * std + mean


def scan_inputs(w: Workload, seed: int = 0, with_h0: bool = False) -> dict:
    """x, delta, A, Bm, Cm, Dv, dy (and optionally h0) as CPU tensors."""
    sd = _store_dtype(w)
    B, L, D, N = w.B, w.L, w.D, w.N
    x = _normal((B, L, D), seed, _X).to(sd)
    z = torch.randn((B, L, D), generator=_gen(seed, _DELTA), dtype=torch.float64)
    z = z * w.delta_sigma + w.delta_mu
    delta = torch.nn.functional.softplus(z).to(sd)
    del z
    A = -torch.arange(1, N + 1, dtype=torch.float32).repeat(D, 1)
    Bm = _normal((B, L, N), seed, _B).to(sd)
    Cm = _normal((B, L, N), seed, _C).to(sd)
    Dv = _param(_normal((D,), seed, _DV), w)
    dy = _normal((B, L, D), seed, _DY).to(sd)
    out = dict(x=x, delta=delta, A=_param(A, w), Bm=Bm, Cm=Cm, Dv=Dv, dy=dy)
    if with_h0:
        out["h0"] = _normal((B, D, N), seed, _H0).contiguous()
    return out


def scan_fused_inputs(w: Workload, seed: int = 0, with_h0: bool = False) -> dict:
    """scan_inputs without delta, plus the inputs of the scan's neighbours in the Mamba
    block: delta_raw [B,L,D] ~ N(0, 1) (the time-step projection's output), delta_bias
    [D] ~ U(-6.9, -2.25) (the bias range that a time step of 1e-3 .. 1e-1 through a
    softplus gives), and the gate input z [B,L,D] ~ N(0, 1).  dy is the upstream gradient
    of the gated output."""
    sd = _store_dtype(w)
    out = scan_inputs(w, seed, with_h0)
    del out["delta"]
    out["delta_raw"] = _normal((w.B, w.L, w.D), seed, _DRAW).to(sd)
    bias = torch.rand((w.D,), generator=_gen(seed, _DBIAS), dtype=torch.float32)
    out["delta_bias"] = _param(bias * (6.9 - 2.25) - 6.9, w)
    out["z"] = _normal((w.B, w.L, w.D), seed, _Z).to(sd)
    return out


def conv_inputs(w: Workload, seed: int = 0) -> dict:
    """x [B,L,D], W [D,K] ~ U(-0.5, 0.5), dout [B,L,D]."""
    sd = _store_dtype(w)
    x = _normal((w.B, w.L, w.D), seed, _CX).to(sd)
    Wc = torch.rand((w.D, w.K), generator=_gen(seed, _CW), dtype=torch.float32) - 0.5
    dout = _normal((w.B, w.L, w.D), seed, _CDOUT).to(sd)
    return dict(x=x, W=_param(Wc, w), dout=dout)


def conv_bias(w: Workload, seed: int = 0) -> torch.Tensor:
    """Conv bias [D] ~ U(-0.5, 0.5) (for the conv forward)."""
    bias = torch.rand((w.D,), generator=_gen(seed, _CBIAS), dtype=torch.float32) - 0.5
    return _param(bias, w)


def rms_inputs(w: Workload, seed: int = 0) -> dict:
    """x, dy [R,M]; scale [M] ~ U(0.5, 1.5).  (The saved rms comes from a forward.)"""
    sd = _store_dtype(w)
    R, M = w.rms_rows, w.rms_dim
    x = _normal((R, M), seed, _RX).to(sd)
    dy = _normal((R, M), seed, _RDY).to(sd)
    scale = torch.rand((M,), generator=_gen(seed, _RSCALE), dtype=torch.float32) + 0.5
    return dict(x=x, dy=dy, scale=_param(scale, w))


def rms_residual(w: Workload, seed: int = 0) -> torch.Tensor:
    """The residual stream [R,M] ~ N(0,1) added before the norm (storage dtype)."""
    return _normal((w.rms_rows, w.rms_dim), seed, _RRES).to(_store_dtype(w))


def as_f64(t: torch.Tensor):
    """Exact f64 copy (numpy) of a stored tensor, for the oracle."""
    return t.to(torch.float64).numpy()


def alpha_inputs(w: Workload, seed: int = 0, with_h0: bool = False) -> dict:
    """Inputs of the sigmoid-gated scan on a workload's shape: batch rows B, steps L,
    state S = N, hidden channels H = D.  The gate and input projections a, b [B,L,N] and
    the upstream gradient dh [B,D] ~ N(0,1), W_c [D,N] ~ U(-0.5, 0.5), and the initial
    hidden state h0 [B,D] zero (the page's zero-initialised h_s2) unless with_h0 (N(0,1)).
    f32 throughout (the page's kernel is f32)."""
    B, L, S, H = w.B, w.L, w.N, w.D
    out = dict(a=_normal((B, L, S), seed, _GA), b=_normal((B, L, S), seed, _GB),
               Wc=torch.rand((H, S), generator=_gen(seed, _GWC), dtype=torch.float32) - 0.5,
               dh=_normal((B, H), seed, _GDH))
    out["h0"] = _normal((B, H), seed, _GH0) if with_h0 else torch.zeros((B, H))
    return out
