"""GPU parity of the conv with its SiLU fused (conv1d_causal_fwd / conv1d_causal_bwd with
act="silu") against the oracle's composition: silu of the oracle's conv forward, and the
oracle's conv backward fed with the oracle's SiLU backward of the upstream gradient.

Small cases are compared on every output (ragged lengths, channel counts that take the
one-channel-per-lane path, every supported conv width, with and without bias).  The full
workloads are compared on a sample of channels (channels are independent).  The fused
backward is also checked against the library's own unfused chain (plain conv forward,
SiLU backward in torch f32, plain conv backward).
"""
import numpy as np
import pytest
import torch

import oracle
from selective_state_space_02_amd import binding as ssm
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import WORKLOADS, custom
from tests.gpu_common import compare, f64, say
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu

CASES = [custom(B=3, L=100, D=20, K=4), custom(B=2, L=37, D=21, K=4, dtype="bf16"),
         custom(B=1, L=5, D=8, K=8), custom(B=2, L=300, D=1028, K=4, dtype="bf16"),
         custom(B=1, L=1000, D=70, K=8, dtype="bf16"), custom(B=2, L=129, D=256, K=4)] + \
        [custom(B=2, L=70, D=12, K=k) for k in (1, 2, 3, 5, 6, 7)]


def ref_fwd(p, bias):
    q = {k: synth.as_f64(v) for k, v in p.items()}
    b = synth.as_f64(bias) if bias is not None else None
    return oracle.silu(oracle.conv1d_fwd(q["x"], q["W"], b))


def ref_bwd(p, bias):
    q = {k: synth.as_f64(v) for k, v in p.items()}
    b = synth.as_f64(bias) if bias is not None else None
    g = oracle.silu_grad(oracle.conv1d_fwd(q["x"], q["W"], b), q["dout"])
    return oracle.conv1d_bwd(q["x"], q["W"], g)


def gpu_both(p, bias):
    g = {k: v.cuda() for k, v in p.items()}
    bg = bias.cuda() if bias is not None else None
    out = ssm.conv1d_causal_fwd(g["x"], g["W"], bg, act="silu")
    r = ssm.conv1d_causal_bwd(g["x"], g["W"], g["dout"], bias=bg, act="silu")
    torch.cuda.synchronize()
    r["out"] = out
    return r


@pytest.mark.parametrize("with_bias", [True, False], ids=["bias", "nobias"])
@pytest.mark.parametrize("w", CASES, ids=lambda w: f"B{w.B}L{w.L}D{w.D}K{w.K}{w.dtype}")
def test_conv_silu_matches_oracle(w, with_bias):
    say(f"[conv silu parity] B={w.B} L={w.L} D={w.D} K={w.K} {w.dtype} bias={with_bias}")
    p = synth.conv_inputs(w)
    bias = synth.conv_bias(w) if with_bias else None
    got = gpu_both(p, bias)
    compare(got, {"out": ref_fwd(p, bias)}, ("out",), label=f"conv silu fwd K={w.K}")
    compare(got, ref_bwd(p, bias), ("dx", "dW", "db"), label=f"conv silu bwd K={w.K}")


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_conv_silu_workloads(w):
    say(f"[conv silu workload] {w.name}")
    p = synth.conv_inputs(w)
    bias = synth.conv_bias(w)
    got = gpu_both(p, bias)
    if w.D > 64:   # channels are independent: check a sample, both ends included
        idx = torch.from_numpy(np.unique(np.concatenate(
            [np.random.default_rng(5).choice(w.D, 40, replace=False), [0, w.D - 1]])))
        p = dict(x=p["x"][:, :, idx].contiguous(), W=p["W"][idx].contiguous(),
                 dout=p["dout"][:, :, idx].contiguous())
        bias = bias[idx].contiguous()
        ic = idx.cuda()
        got = dict(out=got["out"][:, :, ic], dx=got["dx"][:, :, ic], dW=got["dW"][ic],
                   db=got["db"][ic])
    compare(got, {"out": ref_fwd(p, bias)}, ("out",), label=f"conv silu fwd {w.name}")
    compare(got, ref_bwd(p, bias), ("dx", "dW", "db"), label=f"conv silu bwd {w.name}")


def test_plain_backward_ignores_bias():
    # without the activation the gradients do not depend on the bias: it is not read
    w = custom(B=2, L=50, D=24, K=4)
    p = {k: v.cuda() for k, v in synth.conv_inputs(w).items()}
    r0 = ssm.conv1d_causal_bwd(p["x"], p["W"], p["dout"])
    r1 = ssm.conv1d_causal_bwd(p["x"], p["W"], p["dout"], bias=synth.conv_bias(w).cuda())
    torch.cuda.synchronize()
    for k in ("dx", "dW", "db"):
        assert torch.equal(r0[k], r1[k]), k


def test_fused_equals_unfused_chain():
    # f32: the fused backward against plain forward -> SiLU backward (torch, f32) -> plain
    # backward; the two differ only in the rounding of the sigmoid
    w = custom(B=2, L=200, D=64, K=4)
    p = {k: v.cuda() for k, v in synth.conv_inputs(w).items()}
    bias = synth.conv_bias(w).cuda()
    pre = ssm.conv1d_causal_fwd(p["x"], p["W"], bias)
    u = ssm.conv1d_causal_fwd(p["x"], p["W"], bias, act="silu")
    s = torch.sigmoid(pre)
    g = p["dout"] * s * (1.0 + pre * (1.0 - s))
    chain = ssm.conv1d_causal_bwd(p["x"], p["W"], g)
    fused = ssm.conv1d_causal_bwd(p["x"], p["W"], p["dout"], bias=bias, act="silu")
    torch.cuda.synchronize()
    assert rel_err(f64(u), f64(pre * s)) <= 1e-6
    for k in ("dx", "dW", "db"):
        e = rel_err(f64(fused[k]), f64(chain[k]))
        say("fused vs chain", k, f"{e:.2e}")
        assert e <= 1e-5, (k, e)


def test_conv_silu_rows_past_32bit_sizes():
    # D = 50,000,001 f32 channels with K = 8 and SiLU: the rows a workgroup touches span
    # 22 * D * 4 > 2^32 bytes, where a single 32-bit buffer size over all of them would
    # wrap.  Channels are independent, so a sample (first, last, the group boundaries
    # near the end, random ones) is compared with the oracle.
    w = custom(B=1, L=3, D=50_000_001, K=8)
    say(f"[conv silu wide] B={w.B} L={w.L} D={w.D} K={w.K} {w.dtype}")
    p = synth.conv_inputs(w)
    bias = synth.conv_bias(w)
    got = gpu_both(p, bias)
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([[0, 1, 255, 256, w.D - 257, w.D - 256, w.D - 2, w.D - 1],
                                    rng.choice(w.D, 24, replace=False)]))
    t = torch.from_numpy(idx)
    q = dict(x=p["x"][:, :, t].contiguous(), W=p["W"][t].contiguous(),
             dout=p["dout"][:, :, t].contiguous())
    bq = bias[t].contiguous()
    sub = dict(dx=got["dx"][:, :, t.cuda()], dW=got["dW"][t.cuda()], db=got["db"][t.cuda()],
               out=got["out"][:, :, t.cuda()])
    compare(sub, {"out": ref_fwd(q, bq)}, ("out",), label="conv silu fwd wide")
    compare(sub, ref_bwd(q, bq), ("dx", "dW", "db"), label="conv silu bwd wide")
