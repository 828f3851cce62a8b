"""rmsnorm_bwd_noalloc (the allocation-free variant of rmsnorm_bwd, whose scratch is a
static device array) against rmsnorm_bwd with a workspace: two calls in a row on the
shared scratch, the second smaller than the first (so stale partials of the first call
sit in the array), then a row length that takes the looped path; each must equal the
workspace call bit for bit (same plan, kernels and summation order), and the oracle to
the f32 / bf16 tolerances.  A size whose scratch exceeds the array is refused before any
launch, leaving the outputs untouched.  Under HIP graph capture (the callers it is for)
two calls of different shapes, one on the looped path, capture once and replay three
times, with eager work between replays, bit for bit equal to the eager calls."""
import pytest
import torch

from selective_state_space_02_amd import binding as ssm
from selective_state_space_02_amd import synth
from selective_state_space_02_amd.workloads import BY_NAME, custom
from tests.gpu_common import compare, say, with_saved_rms

pytestmark = pytest.mark.gpu

CASES = [BY_NAME["mamba-2.8b"], custom(B=10, L=100, D=777), custom(B=2, L=50, D=9001, dtype="bf16")]


def _both(w):
    p = with_saved_rms(synth.rms_inputs(w, seed=11))
    g = {k: v.cuda() for k, v in p.items()}
    R, M = w.rms_rows, w.rms_dim
    ref = ssm.rmsnorm_bwd(g["dy"], g["x"], g["scale"], g["rms"])
    dx = torch.full_like(g["x"], float("nan"))
    dscale = torch.zeros((M,), dtype=torch.float32, device="cuda")
    got = ssm.rmsnorm_bwd_noalloc(g["dy"], g["x"], g["scale"], g["rms"], dx=dx, dscale=dscale)
    torch.cuda.synchronize()
    return p, got, ref


def test_noalloc_matches_the_workspace_call_twice_in_a_row():
    for i, w in enumerate(CASES):
        say(f"[no-alloc] call {i}: R={w.rms_rows} M={w.rms_dim} {w.dtype}")
        p, got, ref = _both(w)
        assert torch.equal(got["dx"], ref["dx"]), i
        assert torch.equal(got["dscale"], ref["dscale"]), i
        from tests.test_gpu_conv_rms import rms_ref
        compare(got, rms_ref(p), ("dx", "dscale"), label=f"no-alloc call {i}")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    R, M = 32768, 16384  # 512 block partials of 16384 columns: 32 MiB of scratch
    x = torch.zeros((R, M), dtype=torch.bfloat16, device="cuda")
    scale = torch.ones((M,), device="cuda")
    rms = torch.ones((R,), device="cuda")
    dx = torch.full_like(x, 7.0)
    dscale = torch.zeros((M,), device="cuda")
    with pytest.raises(ssm.SsmError) as ei:
        ssm.rmsnorm_bwd_noalloc(x, x, scale, rms, dx=dx, dscale=dscale)
    assert ei.value.code == ssm.SSM_ERR_UNSUPPORTED
    assert "static" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((dx == 7.0).all())  # nothing was launched


def test_noalloc_replays_from_a_graph_bit_identically():
    dev = torch.device("cuda")
    shapes = [custom(B=4, L=64, D=2560, dtype="bf16"), custom(B=3, L=11, D=9001)]
    calls = []
    for w in shapes:
        p = with_saved_rms(synth.rms_inputs(w, seed=12))
        g = {k: v.to(dev) for k, v in p.items()}
        o = dict(dx=torch.empty_like(g["x"]),
                 dscale=torch.zeros((w.rms_dim,), dtype=torch.float32, device=dev))
        calls.append((g, o))

    def run():
        for g, o in calls:
            o["dscale"].zero_()
            ssm.rmsnorm_bwd_noalloc(g["dy"], g["x"], g["scale"], g["rms"], dx=o["dx"],
                                    dscale=o["dscale"])

    run()
    torch.cuda.synchronize()
    ref = [{k: v.clone() for k, v in o.items()} for _, o in calls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        junk = torch.randn(1 << 20, device=dev).sum()
        for _, o in calls:
            o["dx"].fill_(float("nan"))
            o["dscale"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (_, o) in enumerate(calls):
            for k in o:
                assert torch.equal(o[k], ref[i][k]), (rep, i, k)
        say(f"[no-alloc graph] replay {rep} bit-identical ({float(junk):.3f})")

