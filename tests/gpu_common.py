"""Shared code of the GPU parity tests: run the HIP path through the binding, run the
oracle on the same seeded inputs, compare.  Tolerances (normwise max relative error,
max|got-ref| / max|ref|, per output tensor): 1e-4 for f32 paths, the pages' own gradient
tolerance; 2e-2 for outputs stored in bf16.  f32 outputs of bf16-input runs (dA, dB, dC,
dD, dh0, h_last) are held to 1e-4 as well: their inputs are exact bf16 values upcast,
so only f32 arithmetic separates them from the oracle."""
import sys

import numpy as np
import torch

import oracle
from selective_state_space_02_amd import binding as ssm
from selective_state_space_02_amd import synth
from tests.helpers import rel_err

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(t: torch.Tensor) -> float:
    return TOL_BF16 if t.dtype == torch.bfloat16 else TOL_F32


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def scan_gpu(p, use_ckpt=True, with_dh0=True):
    """Run forward then backward on the GPU for CPU input dict p."""
    g = {k: v.cuda() for k, v in p.items()}
    B, L, D = g["x"].shape
    N = g["A"].shape[1]
    ckpt = ssm.new_ckpt(B, L, D, N, g["x"].device) if use_ckpt else None
    h_last = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_scan_fwd(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], h0=g.get("h0"),
                         ckpt=ckpt, h_last=h_last)
    dh0 = torch.empty((B, D, N), dtype=torch.float32, device="cuda") if with_dh0 else None
    r = ssm.ssm_scan_bwd(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], g["dy"],
                         ckpt=ckpt, h0=g.get("h0"), dh0=dh0)
    torch.cuda.synchronize()
    r["y"] = y
    r["h_last"] = h_last
    return r


def scan_oracle(p):
    q = {k: synth.as_f64(v) for k, v in p.items()}
    y, h_last = oracle.scan_fwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], q["Dv"], h0=q.get("h0"))
    r = oracle.scan_bwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], q["Dv"], q["dy"], h0=q.get("h0"))
    r["y"] = y
    r["h_last"] = h_last
    return r


def compare(got: dict, ref: dict, keys, label=""):
    errs = {}
    for k in keys:
        e = rel_err(f64(got[k]), ref[k])
        errs[k] = e
    say(label, " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    for k in keys:
        assert np.isfinite(errs[k]), (label, k)
        assert errs[k] <= tol_for(got[k]), (label, k, errs[k])
    return errs


def with_saved_rms(p: dict) -> dict:
    """RMSNorm inputs plus the statistic the forward saves (from the oracle's forward,
    in f64, stored as the f32 the ABI takes)."""
    _, rms = oracle.rmsnorm_fwd(synth.as_f64(p["x"]), synth.as_f64(p["scale"]), synth.RMS_EPS)
    return dict(p, rms=torch.from_numpy(rms).to(torch.float32))
