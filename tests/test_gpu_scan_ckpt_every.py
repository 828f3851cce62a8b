"""GPU parity of the sparse-checkpoint scan (ssm_scan_fwd_every / ssm_scan_bwd_every):
the forward saves its state every ck_every steps only, and the backward regenerates the
dense states one slab of chunks at a time before its main pass over that slab.

Every output is compared with the oracle on shapes that cover each state size and
storage type, intervals from one tile to longer than the sequence, one and several
slabs (including more slabs than chunks), ragged lengths (a partial last interval and
tile), an initial state, and the backward's own forward recompute (ckpt = NULL).  On
the 2.8B layer the sparse path (64-step interval, 8 slabs) is compared with the dense
path and with the oracle on a sample of channels, and two runs must be bit-identical.
"""
import hashlib

import numpy as np
import pytest
import torch

from selective_state_space_02_amd import binding as ssm
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import BY_NAME, custom
from tests.gpu_common import compare, f64, say, scan_oracle
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

ALL = ("y", "h_last", "dx", "ddelta", "dA", "dB", "dC", "dD", "dh0")

CASES = [
    # name, workload, ck_every, slabs, with_h0, use_ckpt
    ("f32-n16-every16", custom(B=2, L=333, D=80, N=16), 16, 3, False, True),
    ("bf16-n16-every64", custom(B=3, L=500, D=70, N=16, dtype="bf16", delta_mu=-3.0,
                                delta_sigma=1.0), 64, 2, True, True),
    ("f32-n8-every32-recompute", custom(B=2, L=257, D=40, N=8), 32, 4, True, False),
    ("bf16-n4-every48", custom(B=2, L=100, D=24, N=4, dtype="bf16"), 48, 1, True, True),
    ("f32-n16-long-every128", custom(B=1, L=5000, D=64, N=16, delta_mu=-4.0, delta_sigma=1.0),
     128, 5, False, True),
    ("f32-n16-every-beyond-L", custom(B=2, L=70, D=16, N=16), 128, 2, True, True),
    ("bf16-n16-more-slabs-than-chunks", custom(B=2, L=160, D=130, N=16, dtype="bf16"), 32, 50,
     False, True),
    ("f32-n4-every16-recompute", custom(B=3, L=47, D=9, N=4), 16, 2, False, False),
]


def scan_gpu_every(p, ck_every, slabs, use_ckpt=True):
    g = {k: v.cuda() for k, v in p.items()}
    B, L, D = g["x"].shape
    N = g["A"].shape[1]
    ckpt = ssm.new_ckpt(B, L, D, N, g["x"].device, ck_every=ck_every) if use_ckpt else None
    h_last = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_scan_fwd_every(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], ck_every,
                               h0=g.get("h0"), ckpt=ckpt, h_last=h_last)
    dh0 = torch.empty((B, D, N), dtype=torch.float32, device="cuda")
    r = ssm.ssm_scan_bwd_every(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], g["dy"],
                               ck_every, slabs, ckpt=ckpt, h0=g.get("h0"), dh0=dh0)
    torch.cuda.synchronize()
    r["y"] = y
    r["h_last"] = h_last
    return r


@pytest.mark.parametrize("name,w,every,slabs,with_h0,use_ckpt", CASES, ids=[c[0] for c in CASES])
def test_sparse_checkpoints_match_oracle(name, w, every, slabs, with_h0, use_ckpt):
    say(f"[scan every] {name} B={w.B} L={w.L} D={w.D} N={w.N} {w.dtype} every={every} "
        f"slabs={slabs} h0={with_h0} ckpt={use_ckpt}")
    p = synth.scan_inputs(w, seed=5, with_h0=with_h0)
    got = scan_gpu_every(p, every, slabs, use_ckpt=use_ckpt)
    compare(got, scan_oracle(p), ALL, label=name)


def test_checkpoint_bytes_scale_with_the_interval():
    B, L, D, N = 2, 16384, 5120, 16
    dense = ssm.ssm_scan_ckpt_bytes(B, L, D, N)
    assert ssm.ssm_scan_ckpt_bytes_every(B, L, D, N, 0) == dense
    assert ssm.ssm_scan_ckpt_bytes_every(B, L, D, N, 8) == dense
    assert ssm.ssm_scan_ckpt_bytes_every(B, L, D, N, 64) * 8 == dense
    assert ssm.ssm_scan_ckpt_bytes_every(B, L, D, N, 24) == 0     # not a multiple of 16
    assert ssm.ssm_scan_ckpt_bytes_every(2, 100, 8, 4, 8) == 0     # below N = 4's interval


def _digest(r, keys):
    h = hashlib.sha256()
    for k in keys:
        h.update(r[k].detach().cpu().contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def test_sparse_checkpoints_full_workload():
    w = BY_NAME["mamba-2.8b"]
    every, slabs = 64, 8
    say(f"[scan every full] {w.name} every={every} slabs={slabs}: generating inputs")
    p = synth.scan_inputs(w, seed=0)
    g = {k: v.cuda() for k, v in p.items()}
    B, L, D, N = w.B, w.L, w.D, w.N
    ck = ssm.new_ckpt(B, L, D, N, "cuda", ck_every=every)
    assert ck.numel() * 4 * 8 == ssm.ssm_scan_ckpt_bytes(B, L, D, N)
    runs = []
    for i in range(2):
        y = ssm.ssm_scan_fwd_every(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], every,
                                   ckpt=ck)
        r = ssm.ssm_scan_bwd_every(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], g["dy"],
                                   every, slabs, ckpt=ck)
        torch.cuda.synchronize()
        r["y"] = y
        runs.append(r)
        say(f"[scan every full] run {i} done")
    keys = ("y", "dx", "ddelta", "dA", "dB", "dC", "dD")
    assert _digest(runs[0], keys) == _digest(runs[1], keys)
    # the dense path on the same inputs: equal up to summation order (the chunks differ)
    ckd = ssm.new_ckpt(B, L, D, N, "cuda")
    yd = ssm.ssm_scan_fwd(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], ckpt=ckd)
    rd = ssm.ssm_scan_bwd(g["x"], g["delta"], g["A"], g["Bm"], g["Cm"], g["Dv"], g["dy"], ckpt=ckd)
    torch.cuda.synchronize()
    rd["y"] = yd
    got = runs[0]
    errs = {k: rel_err(f64(got[k]), f64(rd[k])) for k in keys}
    say("[scan every full] vs dense: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert torch.equal(got["y"], rd["y"])  # the forward's output does not depend on the interval
    for k in ("dA", "dB", "dC", "dD"):
        assert errs[k] <= 1e-5, (k, errs[k])
    for k in ("dx", "ddelta"):            # bf16 outputs: at most a rounding flip apart
        assert errs[k] <= 2e-2, (k, errs[k])
    # the oracle on a sample of channels (channels are independent in y, dx, ddelta, dA, dD)
    rng = np.random.default_rng(7)
    idx = torch.from_numpy(np.unique(np.concatenate([rng.choice(D, 24, replace=False),
                                                     [0, D - 1]])))
    q = dict(p)
    for k in ("x", "delta", "dy"):
        q[k] = p[k][:, :, idx].contiguous()
    q["A"] = p["A"][idx].contiguous()
    q["Dv"] = p["Dv"][idx].contiguous()
    say(f"[scan every full] oracle on {len(idx)} channels")
    ref = scan_oracle(q)
    sub = {k: got[k][:, :, idx.cuda()] for k in ("y", "dx", "ddelta")}
    sub["dA"] = got["dA"][idx.cuda()]
    sub["dD"] = got["dD"][idx.cuda()]
    compare(sub, ref, ("y", "dx", "ddelta", "dA", "dD"), label="every=64 channels")
