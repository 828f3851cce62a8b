"""The library's calls capture into a HIP graph (through torch.cuda.graph) and replay
correctly: they only launch kernels on the caller's stream (no allocation, copy, memset
or synchronisation inside a call).  One step -- scan forward with checkpoints, scan
backward, conv1d backward with SiLU, RMSNorm backward -- is captured once and replayed
three times, with the program's own eager work and synchronisations between replays;
every replay must reproduce the eager results bit for bit (accumulated outputs are
zeroed eagerly before each run).
"""
import pytest
import torch

from selective_state_space_02_amd import binding as ssm
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import custom
from tests.gpu_common import say

pytestmark = pytest.mark.gpu


def test_step_replays_from_a_graph_bit_identically():
    w = custom(B=2, L=700, D=192, N=16, K=4, dtype="bf16")
    dev = torch.device("cuda")
    p = {k: v.to(dev) for k, v in synth.scan_inputs(w, seed=6).items()}
    c = {k: v.to(dev) for k, v in synth.conv_inputs(w, seed=6).items()}
    r = {k: v.to(dev) for k, v in synth.rms_inputs(w, seed=6).items()}
    cb = synth.conv_bias(w, seed=6).to(dev)
    _, r["rms"] = ssm.rmsnorm_fwd(r["x"], r["scale"], synth.RMS_EPS)
    B, L, D, N, K = w.B, w.L, w.D, w.N, w.K
    code = ssm.SSM_BF16
    f32 = torch.float32
    out = dict(y=torch.empty_like(p["x"]), dx=torch.empty_like(p["x"]),
               ddelta=torch.empty_like(p["x"]), dA=torch.zeros((D, N), dtype=f32, device=dev),
               dB=torch.empty((B, L, N), dtype=f32, device=dev),
               dC=torch.empty((B, L, N), dtype=f32, device=dev),
               dD=torch.zeros((D,), dtype=f32, device=dev), cdx=torch.empty_like(c["x"]),
               dW=torch.zeros((D, K), dtype=f32, device=dev),
               db=torch.zeros((D,), dtype=f32, device=dev), rdx=torch.empty_like(r["x"]),
               dscale=torch.zeros((w.rms_dim,), dtype=f32, device=dev))
    ckpt = ssm.new_ckpt(B, L, D, N, dev)
    u8 = torch.uint8
    ws_f = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(B, L, D, N, code)), dtype=u8, device=dev)
    ws_b = torch.empty(max(1, ssm.ssm_scan_bwd_workspace_bytes(B, L, D, N, code, True)), dtype=u8, device=dev)
    ws_c = torch.empty(max(1, ssm.conv1d_causal_bwd_workspace_bytes(B, L, D, K, code)), dtype=u8, device=dev)
    ws_r = torch.empty(max(1, ssm.rmsnorm_bwd_workspace_bytes(w.rms_rows, w.rms_dim, code)), dtype=u8, device=dev)
    accum = ("dA", "dD", "dW", "db", "dscale")

    def step():
        ssm.ssm_scan_fwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], y=out["y"],
                         ckpt=ckpt, ws=ws_f)
        ssm.ssm_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], p["dy"],
                         ckpt=ckpt, dx=out["dx"], ddelta=out["ddelta"], dA=out["dA"],
                         dB=out["dB"], dC=out["dC"], dD=out["dD"], ws=ws_b)
        ssm.conv1d_causal_bwd(c["x"], c["W"], c["dout"], bias=cb, act="silu", dx=out["cdx"],
                              dW=out["dW"], db=out["db"], ws=ws_c)
        ssm.rmsnorm_bwd(r["dy"], r["x"], r["scale"], r["rms"], dx=out["rdx"],
                        dscale=out["dscale"], ws=ws_r)

    def zero_accumulators():
        for k in accum:
            out[k].zero_()

    # eager reference
    zero_accumulators()
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}

    # capture (on torch's capture stream, which the binding passes to the library)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        zero_accumulators()
        step()  # warm-up on the side stream, as torch recommends before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    zero_accumulators()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        # the program's own eager work between replays
        junk = torch.randn(1 << 20, device=dev).sum()
        for k in out:  # overwritten outputs must be rewritten by the replay
            if k not in accum:
                out[k].fill_(float("nan"))
        zero_accumulators()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (rep, k)
        say(f"[graph] replay {rep} bit-identical ({float(junk):.3f})")


def test_sparse_checkpoint_scan_replays_from_a_graph_bit_identically():
    # the sparse-checkpoint path launches per slab (regeneration, then the main pass);
    # the forward, and the backward with a final-state gradient, are captured together
    w = custom(B=2, L=700, D=130, N=16, dtype="bf16")
    dev = torch.device("cuda")
    p = {k: v.to(dev) for k, v in synth.scan_inputs(w, seed=8).items()}
    B, L, D, N = w.B, w.L, w.D, w.N
    f32 = torch.float32
    every, slabs = 64, 3
    code = ssm.SSM_BF16
    u8 = torch.uint8
    ckpt = ssm.new_ckpt(B, L, D, N, dev, ck_every=every)
    ws_f = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(B, L, D, N, code)), dtype=u8, device=dev)
    ws_b = torch.empty(max(1, ssm.ssm_scan_bwd_workspace_bytes_every(B, L, D, N, code, True, every, slabs)),
                       dtype=u8, device=dev)
    dh_last = torch.randn((B, D, N), dtype=f32, device=dev)
    out = dict(y=torch.empty_like(p["x"]), dx=torch.empty_like(p["x"]), ddelta=torch.empty_like(p["x"]),
               dA=torch.zeros((D, N), dtype=f32, device=dev), dB=torch.empty((B, L, N), dtype=f32, device=dev),
               dC=torch.empty((B, L, N), dtype=f32, device=dev), dD=torch.zeros((D,), dtype=f32, device=dev),
               dh0=torch.empty((B, D, N), dtype=f32, device=dev))
    a = (p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"])

    def run():
        out["dA"].zero_()
        out["dD"].zero_()
        ssm.ssm_scan_fwd_every(*a, every, y=out["y"], ckpt=ckpt, ws=ws_f)
        ssm.ssm_scan_bwd_every(*a, p["dy"], every, slabs, ckpt=ckpt, dx=out["dx"],
                               ddelta=out["ddelta"], dA=out["dA"], dB=out["dB"], dC=out["dC"],
                               dD=out["dD"], dh0=out["dh0"], dh_last=dh_last, ws=ws_b)

    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        junk = torch.randn(1 << 20, device=dev).sum()
        for k in out:
            out[k].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (rep, k)
        say(f"[graph sparse] replay {rep} bit-identical ({float(junk):.3f})")
