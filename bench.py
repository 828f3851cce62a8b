"""Benchmark of the selective-scan hot path on one MI355X.

A step is one pass of the whole path over one batch of seeded synthetic input already
resident in HBM: ssm_scan_fwd (with checkpoints), ssm_scan_bwd, conv1d_causal_bwd and
rmsnorm_bwd, each through the C ABI.  Default workload: the Mamba-2.8B-shaped layer
(B=2, L=16384, d_inner=5120, d_state=16, d_conv=4, bf16 activations, f32 state and
arithmetic; RMSNorm backward over [32768, 2560]).

Prints one JSON line.  `value` is the metric the workload is quoted on: tokens*channels
per second of the scan forward+backward: B*L*D over the time per (forward, backward)
pair, the pairs called back to back with one HIP event pair around them all on the stream
they run on.  The whole step's rate, and a per-call and per-kernel breakdown from an
instrumented loop (events around every call and around the timed kernels), are reported
beside it.  The
`roofline` entry covers the dominant kernel (the backward main pass): its algorithmic
HBM bytes per launch over its average launch time (HIP events recorded by the library
around that kernel on its own stream) against the 8 TB/s HBM peak, and, beside that, its
VALU issue time from the committed counter record against its measured time.  The f64
CPU oracle is timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --gpus N        (N > 1 exits: the scan library runs on one GPU)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scan fwd+bwd tokens·channels/sec and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0

# MI355X VALU issue: 256 CUs x 4 SIMDs; a SIMD issues one wave64 VALU instruction per 4
# cycles (16 lanes per cycle) at 2.4 GHz, and a transcendental one (v_exp_f32) occupies
# it for 8 (the counter record's SQ_ACTIVE_INST_VALU equals 4 cycles per VALU instruction
# plus 4 more per transcendental one to within 1.3%).  Without packed f32 (disabled in
# every build) that is 3.93e13 lane-operations/s, or 78.6 TFLOP/s counting an FMA as 2.
SIMDS = 256 * 4
CLOCK_HZ = 2.4e9
VALU_WAVE_INSTR_PER_S = SIMDS * CLOCK_HZ / 4
LANE_OPS_PEAK = VALU_WAVE_INSTR_PER_S * 64
FP32_NONPACKED_PEAK_TFLOPS = 2 * LANE_OPS_PEAK / 1e12

# Operations the backward main pass must issue per state update (b, t, d, n), as the
# method's cost model counts them: recompute of a_t and h_t (delta*A, exp, delta*x*B,
# state FMA) and the reverse step (g = dy*C + g', a*h_{t-1}, g*q, the dA FMA, the
# sum g*A*q, the sum g*B, the dB term g*delta*x, the dC term dy*h, the carry a*g):
# 13 VALU operations and 1 exp.  The cross-lane channel sums come on top.
BWD_MAIN_VALU_PER_UPDATE = 13
BWD_MAIN_EXP_PER_UPDATE = 1


class HipEvents:
    """Raw hipEvent_t pairs (the library's timing hook records them itself, so they are
    created and read through the HIP runtime directly)."""

    def __init__(self):
        import ctypes
        self.c = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipGetLastError.argtypes = []
        self.made = []

    def pair(self):
        a, b = self.c.c_void_p(), self.c.c_void_p()
        assert self.hip.hipEventCreate(self.c.byref(a)) == 0
        assert self.hip.hipEventCreate(self.c.byref(b)) == 0
        self.made += [a.value, b.value]
        return a.value, b.value

    def record(self, ev, stream_handle):
        assert self.hip.hipEventRecord(self.c.c_void_p(ev), self.c.c_void_p(stream_handle)) == 0

    def elapsed_ms(self, start, stop):
        """None if the pair was never recorded (a kernel the workload did not launch)."""
        ms = self.c.c_float()
        rc = self.hip.hipEventElapsedTime(self.c.byref(ms), self.c.c_void_p(start), self.c.c_void_p(stop))
        if rc != 0:
            self.hip.hipGetLastError()  # the query's own error, not left pending for later calls
            return None
        return ms.value

    def destroy(self):
        for e in self.made:
            self.hip.hipEventDestroy(self.c.c_void_p(e))
        self.made = []


BWD_MAIN_SOURCES = ("scan_bwd.hip", "common.hpp", "tile.hpp", "launch.hpp")
COUNTERS_MD = os.path.join(ROOT, "profiles", "k_bwd_main_mamba-2.8b_counters.md")


def bwd_main_source_hash():
    """sha256 over the sources that define the backward main kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in BWD_MAIN_SOURCES:
        h.update(open(os.path.join(ROOT, "selective_state_space_02_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def counter_record(workload_name):
    """The backward main kernel's record in the committed rocprofv3 counter summary, or
    None when there is none for this workload or the kernel's sources changed since the
    counters were taken."""
    if workload_name != "mamba-2.8b" or not os.path.exists(COUNTERS_MD):
        return None
    text = open(COUNTERS_MD).read()
    if "```json" not in text:
        return None
    rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    if rec.get("source_sha256") != bwd_main_source_hash():
        return None
    return rec


def counter_traffic(workload_name):
    """HBM bytes per launch of the backward main kernel from the FETCH_SIZE/WRITE_SIZE
    counters (copy-calibrated), or None (see counter_record)."""
    rec = counter_record(workload_name)
    return rec.get("traffic_bytes_per_launch") if rec else None


def counter_valu_slots(workload_name):
    """VALU issue slots per launch of the backward main kernel from the committed counter
    record: wave64 VALU instructions, a transcendental one counting twice (SQ_INSTS_VALU
    + SQ_INSTS_VALU_TRANS_F32), or None (see counter_record)."""
    rec = counter_record(workload_name)
    if not rec:
        return None
    sq = rec["sq"]
    return sq["SQ_INSTS_VALU"] + sq["SQ_INSTS_VALU_TRANS_F32"]


def algorithmic_bytes(w):
    """Bytes the method must move per step (HBM), by operation."""
    s = 2 if w.dtype == "bf16" else 4
    E = w.B * w.L * w.D
    P = w.B * w.L * w.N
    DN = w.D * w.N
    fwd = 3 * E * s + 2 * P * s + (DN + w.D) * 4
    bwd = 5 * E * s + 2 * P * s + 2 * P * 4 + 3 * (DN + w.D) * 4
    conv = 3 * E * s + w.D * w.K * 4 * 3 + w.D * 4 * 2
    RM = w.rms_rows * w.rms_dim
    rms = 3 * RM * s + w.rms_dim * 4 * 3 + w.rms_rows * 4
    return dict(scan_fwd=fwd, scan_bwd=bwd, conv_bwd=conv, rms_bwd=rms)


def bwd_main_bytes(w):
    """Algorithmic HBM bytes of the backward main kernel alone: x, delta, dy, B, C read;
    dx, ddelta written (the dB/dC/dA/dD sums leave through the reduction kernels)."""
    s = 2 if w.dtype == "bf16" else 4
    E = w.B * w.L * w.D
    P = w.B * w.L * w.N
    return 5 * E * s + 2 * P * s


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, cpu_inputs, sample_channels, budget_note):
    """The f64 oracle on a bounded sample: the scan forward+backward and the conv1d
    backward on `sample_channels` channels (all batch rows, full length), and the
    RMSNorm backward on the same fraction of its rows.  Scaled to tokens*channels/s of
    the sample."""
    import oracle
    from selective_state_space_02_amd import synth

    frac = sample_channels / w.D
    p, c, r = cpu_inputs
    q = {}
    for k in ("x", "delta", "dy"):
        q[k] = synth.as_f64(p[k][:, :, :sample_channels].contiguous())
    q["A"] = synth.as_f64(p["A"][:sample_channels].contiguous())
    q["Dv"] = synth.as_f64(p["Dv"][:sample_channels].contiguous())
    q["Bm"] = synth.as_f64(p["Bm"])
    q["Cm"] = synth.as_f64(p["Cm"])
    cq = {k: synth.as_f64(v[..., :sample_channels].contiguous() if v.dim() == 3 else
                          v[:sample_channels].contiguous()) for k, v in c.items()}
    nrows = max(1, int(round(w.rms_rows * frac)))
    rq = {"x": synth.as_f64(r["x"][:nrows]), "dy": synth.as_f64(r["dy"][:nrows]),
          "scale": synth.as_f64(r["scale"])}
    _, rq["rms"] = oracle.rmsnorm_fwd(rq["x"], rq["scale"], synth.RMS_EPS)  # saved statistic
    t0 = time.perf_counter()
    oracle.scan_fwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], q["Dv"])
    oracle.scan_bwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], q["Dv"], q["dy"])
    t1 = time.perf_counter()
    oracle.conv1d_bwd(cq["x"], cq["W"], cq["dout"])
    t2 = time.perf_counter()
    oracle.rmsnorm_bwd(rq["dy"], rq["x"], rq["scale"], rq["rms"])
    t3 = time.perf_counter()
    tokch = w.B * w.L * sample_channels
    return {
        "value": tokch / (t3 - t0),
        "unit": "tokens*channels/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{sample_channels} of {w.D} channels (all {w.B} batch rows x {w.L} steps) "
                   f"for the scan fwd+bwd and conv1d bwd, {nrows} of {w.rms_rows} rows for the "
                   f"RMSNorm bwd; f64; {budget_note}"),
        "seconds": {"scan_fwd_bwd": t1 - t0, "conv_bwd": t2 - t1, "rms_bwd": t3 - t2},
    }


def measure_layer_forward(w, c, r, seed, steps, dev):
    """The layer-forward kernels around the scan (conv1d and RMSNorm forward, the latter
    also with the residual stream added first) on the workload's shapes, timed with the
    library's timing hook over `steps` launches each.
    Not part of the step and not in `value`; both are HBM-bound, so each reports its
    algorithmic bytes (read the input once, write the output once) per second."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    f32 = torch.float32
    s = 2 if w.dtype == "bf16" else 4
    cout = torch.empty_like(c["x"])
    cbias = synth.conv_bias(w, seed).to(dev)
    ry = torch.empty_like(r["x"])
    rrms = torch.empty((w.rms_rows,), dtype=f32, device=dev)

    def run():
        ssm.conv1d_causal_fwd(c["x"], c["W"], cbias, out=cout)
        ssm.rmsnorm_fwd(r["x"], r["scale"], synth.RMS_EPS, y=ry, rms=rrms)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    he = HipEvents()
    names = ("conv_fwd", "rms_fwd")
    kev = {k: [he.pair() for _ in range(steps)] for k in names}
    for i in range(steps):
        for k in names:
            ssm.ssm_set_kernel_timer(k, *kev[k][i])
        run()
    torch.cuda.synchronize()
    for k in names:
        ssm.ssm_set_kernel_timer(k, None, None)
    ms = {k: sum(he.elapsed_ms(*pr) for pr in kev[k]) / steps for k in names}
    # the norm with the residual stream added first (reads x and residual, writes y and
    # the summed stream)
    rres = synth.rms_residual(w, seed).to(dev)
    rout = torch.empty_like(r["x"])

    def run_res():
        ssm.rmsnorm_fwd(r["x"], r["scale"], synth.RMS_EPS, y=ry, rms=rrms, residual=rres,
                        residual_out=rout)
    for _ in range(2):
        run_res()
    torch.cuda.synchronize()
    rev = [he.pair() for _ in range(steps)]
    for i in range(steps):
        ssm.ssm_set_kernel_timer("rms_fwd", *rev[i])
        run_res()
    torch.cuda.synchronize()
    ssm.ssm_set_kernel_timer("rms_fwd", None, None)
    ms["rms_fwd_residual"] = sum(he.elapsed_ms(*pr) for pr in rev) / steps
    names = names + ("rms_fwd_residual",)
    he.destroy()
    E = w.B * w.L * w.D
    RM = w.rms_rows * w.rms_dim
    nbytes = {"conv_fwd": 2 * E * s + w.D * (w.K + 1) * 4,
              "rms_fwd": 2 * RM * s + (w.rms_dim + w.rms_rows) * 4,
              "rms_fwd_residual": 4 * RM * s + (w.rms_dim + w.rms_rows) * 4}
    out = {}
    for k in names:
        gbps = nbytes[k] / (ms[k] * 1e-3) / 1e9
        out[k] = {"kernel_ms": ms[k], "algorithmic_bytes": nbytes[k], "GBps": gbps,
                  "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS}
    return out


def measure_conv_silu(w, c, seed, steps, dev):
    """The conv with its SiLU fused (act="silu"), forward and backward, on the workload's
    shapes, timed with the library's timing hook over `steps` launches each (the backward
    figure is its main kernel; the dW/db partial reduction is as in the plain backward).
    Not part of the step and not in `value`.  The fused kernels move the same algorithmic
    bytes as the plain ones; an unfused chain would add a SiLU pass (read, write) after
    the forward and a SiLU-backward pass (read du and the conv output, write g) before
    the backward, counted in `unfused_extra_bytes`."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    f32 = torch.float32
    s = 2 if w.dtype == "bf16" else 4
    D, K = w.D, w.K
    bias = synth.conv_bias(w, seed).to(dev)
    out = torch.empty_like(c["x"])
    dx = torch.empty_like(c["x"])
    dW = torch.zeros((D, K), dtype=f32, device=dev)
    db = torch.zeros((D,), dtype=f32, device=dev)
    code = 1 if w.dtype == "bf16" else 0
    ws = torch.empty(max(1, ssm.conv1d_causal_bwd_workspace_bytes(w.B, w.L, D, K, code)),
                     dtype=torch.uint8, device=dev)

    def run():
        ssm.conv1d_causal_fwd(c["x"], c["W"], bias, act="silu", out=out)
        ssm.conv1d_causal_bwd(c["x"], c["W"], c["dout"], bias=bias, act="silu", dx=dx, dW=dW,
                              db=db, ws=ws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    he = HipEvents()
    names = ("conv_fwd", "conv_bwd")
    kev = {k: [he.pair() for _ in range(steps)] for k in names}
    for i in range(steps):
        for k in names:
            ssm.ssm_set_kernel_timer(k, *kev[k][i])
        run()
    torch.cuda.synchronize()
    for k in names:
        ssm.ssm_set_kernel_timer(k, None, None)
    ms = {k: sum(he.elapsed_ms(*pr) for pr in kev[k]) / steps for k in names}
    he.destroy()
    E = w.B * w.L * D
    nbytes = {"conv_fwd": 2 * E * s + D * (K + 1) * 4, "conv_bwd": 3 * E * s + D * (K + 1) * 4}
    extra = {"conv_fwd": 2 * E * s, "conv_bwd": 3 * E * s}
    res = {}
    for k in names:
        gbps = nbytes[k] / (ms[k] * 1e-3) / 1e9
        res[k + "_silu"] = {"kernel_ms": ms[k], "algorithmic_bytes": nbytes[k], "GBps": gbps,
                            "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
                            "unfused_extra_bytes": extra[k]}
    return res


def measure_scan_fused(w, seed, steps, dev):
    """The scan with its Mamba-block neighbours fused in (ssm_scan_fused_fwd/bwd: time
    step softplus(delta + bias), output gate y * silu(z)) on the workload's shapes, each
    call timed with events on the stream it is launched on, over `steps` calls.  Not part
    of the step and not in `value`.  The fused calls move the plain scan's bytes plus the
    gate's (z read by the forward, the backward's summary and main passes; y before the
    gate written and read back; dz written).  Separate elementwise passes around the plain
    scan would instead move `unfused_extra_bytes` (forward: softplus read+write, gate two
    reads + write; backward: gate backward three reads + two writes, softplus backward two
    reads + write, bias sum one read), whose time at the HBM peak is a lower bound on what
    they would cost."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    f32 = torch.float32
    code = ssm.SSM_BF16 if w.dtype == "bf16" else ssm.SSM_F32
    B, L, D, N = w.B, w.L, w.D, w.N
    g = {k: v.to(dev) for k, v in synth.scan_fused_inputs(w, seed).items()}
    out = torch.empty_like(g["x"])
    ysave = torch.empty_like(g["x"])
    ckpt = ssm.new_ckpt(B, L, D, N, dev)
    ws_f = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(B, L, D, N, code)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, ssm.ssm_scan_bwd_workspace_bytes(B, L, D, N, code, True)), dtype=torch.uint8, device=dev)
    grads = dict(dx=torch.empty_like(g["x"]), ddelta=torch.empty_like(g["x"]),
                 dA=torch.zeros((D, N), dtype=f32, device=dev),
                 dB=torch.empty((B, L, N), dtype=f32, device=dev),
                 dC=torch.empty((B, L, N), dtype=f32, device=dev),
                 dD=torch.zeros((D,), dtype=f32, device=dev), dz=torch.empty_like(g["x"]),
                 ddelta_bias=torch.zeros((D,), dtype=f32, device=dev))
    kw = dict(delta_bias=g["delta_bias"], delta_softplus=True, z=g["z"])
    args = (g["x"], g["delta_raw"], g["A"], g["Bm"], g["Cm"], g["Dv"])

    def fwd():
        ssm.ssm_scan_fused_fwd(*args, out=out, y_save=ysave, ckpt=ckpt, ws=ws_f, **kw)

    def bwd():
        ssm.ssm_scan_fused_bwd(*args, g["dy"], ckpt=ckpt, y_save=ysave, ws=ws_b, **kw, **grads)
    for _ in range(2):
        fwd()
        bwd()
    torch.cuda.synchronize()
    he = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = {k: [he.pair() for _ in range(steps)] for k in ("fused_fwd", "fused_bwd")}
    knames = ("fwd_summary", "fwd_output", "bwd_summary", "bwd_main")
    kev = {k: [he.pair() for _ in range(steps)] for k in knames}
    for i in range(steps):
        for k in knames:
            ssm.ssm_set_kernel_timer(k, *kev[k][i])
        for k, f in (("fused_fwd", fwd), ("fused_bwd", bwd)):
            he.record(ev[k][i][0], stream)
            f()
            he.record(ev[k][i][1], stream)
    torch.cuda.synchronize()
    for k in knames:
        ssm.ssm_set_kernel_timer(k, None, None)
    ms = {k: sum(he.elapsed_ms(*pr) for pr in ev[k]) / steps for k in ev}
    kms = {}
    for k in knames:
        vals = [he.elapsed_ms(*pr) for pr in kev[k]]
        kms[k] = None if any(v is None for v in vals) else sum(vals) / steps
    he.destroy()
    s = 2 if w.dtype == "bf16" else 4
    E = B * L * D * s
    extra = 2 * E + 3 * E + (5 * E + 3 * E + E)
    return {"call_ms": ms, "kernel_ms": kms,
            "tokens_channels_per_s": B * L * D / ((ms["fused_fwd"] + ms["fused_bwd"]) * 1e-3),
            "fused_extra_bytes": 6 * E, "unfused_extra_bytes": extra,
            "unfused_extra_ms_at_hbm_peak": extra / (HBM_PEAK_GBPS * 1e9) * 1e3}


# Checkpoint intervals measured beside the step, with the slabs the sparse backward
# regenerates its dense states in: (interval in steps, slabs); 0 is the default interval
# (8 steps at N = 16), 512 the backward's chunk length on the 2.8B layer (a state at
# each chunk start only).
CKPT_INTERVALS = ((0, 1), (16, 4), (64, 2), (64, 8), (512, 4))


def measure_ckpt_intervals(w, p, steps, dev):
    """The scan forward and backward with the forward's states saved every `every` steps
    (ssm_scan_fwd_every / ssm_scan_bwd_every; the backward regenerates the dense states of
    one slab at a time), timed per call with events on the stream, against the checkpoint
    memory and the backward's workspace.  Not part of the step and not in `value`."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    f32 = torch.float32
    code = ssm.SSM_BF16 if w.dtype == "bf16" else ssm.SSM_F32
    B, L, D, N = w.B, w.L, w.D, w.N
    y = torch.empty_like(p["x"])
    g = dict(dx=torch.empty_like(p["x"]), ddelta=torch.empty_like(p["x"]),
             dA=torch.zeros((D, N), dtype=f32, device=dev), dB=torch.empty((B, L, N), dtype=f32, device=dev),
             dC=torch.empty((B, L, N), dtype=f32, device=dev), dD=torch.zeros((D,), dtype=f32, device=dev))
    ws_f = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(B, L, D, N, code)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = {}
    for every, slabs in CKPT_INTERVALS:
        ck = ssm.new_ckpt(B, L, D, N, dev, ck_every=every)
        wsb = ssm.ssm_scan_bwd_workspace_bytes_every(B, L, D, N, code, True, every, slabs)
        ws_b = torch.empty(max(1, wsb), dtype=torch.uint8, device=dev)

        def fwd():
            ssm.ssm_scan_fwd_every(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], every,
                                   y=y, ckpt=ck, ws=ws_f)

        def bwd():
            ssm.ssm_scan_bwd_every(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], p["dy"],
                                   every, slabs, ckpt=ck, ws=ws_b, **g)
        for _ in range(2):
            fwd()
            bwd()
        torch.cuda.synchronize()
        he = HipEvents()
        ev = {k: [he.pair() for _ in range(steps)] for k in ("fwd", "bwd")}
        kev = [he.pair() for _ in range(steps)]
        for i in range(steps):
            ssm.ssm_set_kernel_timer("fwd_output", *kev[i])
            for k, f in (("fwd", fwd), ("bwd", bwd)):
                he.record(ev[k][i][0], stream)
                f()
                he.record(ev[k][i][1], stream)
        torch.cuda.synchronize()
        ssm.ssm_set_kernel_timer("fwd_output", None, None)
        ms = {k: sum(he.elapsed_ms(*pr) for pr in ev[k]) / steps for k in ev}
        fo = sum(he.elapsed_ms(*pr) for pr in kev) / steps
        he.destroy()
        label = f"every {every} slabs {slabs}" if every else f"every {8 if N == 16 else 16} (default)"
        out[label] = {"slabs": slabs, "ckpt_bytes": ck.numel() * 4, "bwd_workspace_bytes": wsb,
                      "fwd_ms": ms["fwd"], "fwd_output_kernel_ms": fo, "bwd_ms": ms["bwd"],
                      "fwd_bwd_ms": ms["fwd"] + ms["bwd"]}
        del ck, ws_b
        torch.cuda.empty_cache()
    return out


def measure_alpha_scan(seed, steps, dev):
    """The sigmoid-gated scan (ssm_alpha_scan_fwd/bwd) on the shape of the pages' alpha
    stack (256 sequences of 32 steps, state 16, hidden 64), each call timed with events on
    its stream.  Not part of the step and not in `value`.  Algorithmic bytes: the forward
    reads a, b, W_c, h0 and writes h; the backward reads a, b, W_c, dh and writes da, db,
    dh0 and dW_c (read and written)."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    from selective_state_space_02_amd.workloads import BY_NAME
    w = BY_NAME["alpha-stack"]
    Bn, K, S, H = w.B, w.L, w.N, w.D
    p = {k: v.to(dev) for k, v in synth.alpha_inputs(w, seed).items()}
    h = torch.empty((Bn, H), device=dev)
    g = dict(da=torch.empty_like(p["a"]), db=torch.empty_like(p["b"]),
             dWc=torch.zeros_like(p["Wc"]), dh0=torch.empty((Bn, H), device=dev))
    ws = torch.empty(max(1, int(ssm.load().ssm_alpha_scan_bwd_workspace_bytes(Bn, K, S, H))),
                     dtype=torch.uint8, device=dev)

    def fwd():
        ssm.ssm_alpha_scan_fwd(p["a"], p["b"], p["Wc"], h0=p["h0"], h=h)

    def bwd():
        ssm.ssm_alpha_scan_bwd(p["a"], p["b"], p["Wc"], p["dh"], ws=ws, **g)
    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    he = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = {k: [he.pair() for _ in range(steps)] for k in ("fwd", "bwd")}
    for i in range(steps):
        for k, f in (("fwd", fwd), ("bwd", bwd)):
            he.record(ev[k][i][0], stream)
            f()
            he.record(ev[k][i][1], stream)
    torch.cuda.synchronize()
    ms = {k: sum(he.elapsed_ms(*pr) for pr in ev[k]) / steps for k in ev}
    he.destroy()
    P, Hb, W = Bn * K * S * 4, Bn * H * 4, H * S * 4
    nbytes = {"fwd": 2 * P + W + 2 * Hb, "bwd": 4 * P + 2 * W + 2 * Hb + 2 * W}
    return {"shape": {"Bn": Bn, "K": K, "S": S, "H": H}, "fwd_ms": ms["fwd"], "bwd_ms": ms["bwd"],
            "algorithmic_bytes": nbytes,
            "GBps": {k: nbytes[k] / (ms[k] * 1e-3) / 1e9 for k in ms}}


def measure_scan_back_to_back(call_fwd, call_bwd, steps):
    """The scan forward and backward called back to back `steps` times with one event
    pair around them all, on the stream the calls launch on: the metric's time.  No event
    sits between the kernels (each one recorded there leaves the GPU idle for a few
    microseconds; the instrumented loop that gives the per-call and per-kernel breakdown
    records about ten per scan step)."""
    import torch
    for _ in range(2):
        call_fwd()
        call_bwd()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        call_fwd()
        call_bwd()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure_graph_step(calls, steps, dev):
    """The step's library calls captured once into a HIP graph (torch.cuda.graph; the
    calls only launch kernels on the caller's stream) and replayed: the time per step
    of `steps` replays against `steps` eager steps, both bracketed by events on the
    current stream.  The difference, if any, is what the launch path costs the eager
    steps.  Not part of `value`."""
    import torch

    def step():
        for _, f in calls:
            f()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    g.replay()
    eager_ms = timed(step)
    graph_ms = timed(g.replay)
    return {"eager_ms": eager_ms, "graph_ms": graph_ms, "steps": steps}


def measure_copy_GBps(dev, reps=5):
    """A plain 1 GiB device-to-device copy (torch's copy on the current stream), timed
    with events: the practical HBM rate the bandwidth fractions are also quoted against
    (read + write bytes per second)."""
    import torch
    a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    he = HipEvents()
    st = torch.cuda.current_stream(dev).cuda_stream
    pairs = [he.pair() for _ in range(reps)]
    for pr in pairs:
        he.record(pr[0], st)
        b.copy_(a)
        he.record(pr[1], st)
    torch.cuda.synchronize()
    ms = sorted(he.elapsed_ms(*pr) for pr in pairs)[reps // 2]
    he.destroy()
    del a, b
    return 2 * (1 << 30) / (ms * 1e-3) / 1e9


# Sequences decoded together: a serving batch whose f32 state (1024 x 5120 x 16 x 4 B =
# 335 MB on the 2.8B layer) exceeds the 256 MB Infinity Cache, so the scan step's rate
# is an HBM rate (at 256 sequences the 84 MB state stays cache-resident across tokens).
DECODE_BATCH = 1024


def measure_decode(w, seed, steps, dev):
    """One-token decode (conv1d_causal_step then ssm_scan_step) for DECODE_BATCH
    sequences at the workload's D, N, K, timed with the library's timing hook over `steps`
    tokens.  Not part of the step and not in `value`.  Both kernels are HBM-bound: the
    scan step reads and writes its f32 state, the conv step its window."""
    import torch
    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    from selective_state_space_02_amd.workloads import custom
    wd = custom(B=DECODE_BATCH, L=1, D=w.D, N=w.N, K=w.K, dtype=w.dtype)
    p = {k: v.to(dev) for k, v in synth.scan_inputs(wd, seed, with_h0=True).items()}
    c = {k: v.to(dev) for k, v in synth.conv_inputs(wd, seed).items()}
    bias = synth.conv_bias(wd, seed).to(dev)
    Bd, D, N, K = DECODE_BATCH, w.D, w.N, w.K
    h = p["h0"].clone()
    state = torch.zeros((Bd, K - 1, D), dtype=c["x"].dtype, device=dev)
    xt, dt = p["x"][:, 0].contiguous(), p["delta"][:, 0].contiguous()
    bt, ct = p["Bm"][:, 0].contiguous(), p["Cm"][:, 0].contiguous()
    cx = c["x"][:, 0].contiguous()
    cout = torch.empty_like(cx)
    yt = torch.empty_like(xt)

    def token():
        ssm.conv1d_causal_step(state, cx, c["W"], bias, out_t=cout)
        ssm.ssm_scan_step(h, xt, dt, p["A"], bt, ct, p["Dv"], y_t=yt)
    for _ in range(3):
        token()
    torch.cuda.synchronize()
    he = HipEvents()
    names = ("conv_step", "scan_step")
    kev = {k: [he.pair() for _ in range(steps)] for k in names}
    tev = [he.pair() for _ in range(steps)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(steps):
        for k in names:
            ssm.ssm_set_kernel_timer(k, *kev[k][i])
        he.record(tev[i][0], stream)
        token()
        he.record(tev[i][1], stream)
    torch.cuda.synchronize()
    for k in names:
        ssm.ssm_set_kernel_timer(k, None, None)
    ms = {k: sum(he.elapsed_ms(*pr) for pr in kev[k]) / steps for k in names}
    tok_ms = sum(he.elapsed_ms(*pr) for pr in tev) / steps
    he.destroy()
    s = 2 if w.dtype == "bf16" else 4
    nbytes = {"scan_step": 2 * Bd * D * N * 4 + 3 * Bd * D * s + 2 * Bd * N * s + D * (N + 1) * 4,
              "conv_step": 2 * Bd * (K - 1) * D * s + 2 * Bd * D * s + D * (K + 1) * 4}
    out = {"batch": Bd, "token_ms": tok_ms, "tokens_per_s": Bd / (tok_ms * 1e-3)}
    for k in names:
        gbps = nbytes[k] / (ms[k] * 1e-3) / 1e9
        out[k] = {"kernel_ms": ms[k], "algorithmic_bytes": nbytes[k], "GBps": gbps,
                  "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS}

    # the Mamba block's token: conv step with its SiLU, then the fused scan step (time
    # step softplus(delta + bias), output gate silu(z)), still two launches
    f = {k: v.to(dev) for k, v in synth.scan_fused_inputs(wd, seed, with_h0=True).items()}
    hf = f["h0"].clone()
    ft = {k: f[k][:, 0].contiguous() for k in ("x", "delta_raw", "Bm", "Cm", "z")}

    def fused_token():
        ssm.conv1d_causal_step(state, cx, c["W"], bias, act="silu", out_t=cout)
        ssm.ssm_scan_fused_step(hf, ft["x"], ft["delta_raw"], f["A"], ft["Bm"], ft["Cm"], f["Dv"],
                                delta_bias=f["delta_bias"], delta_softplus=True, z_t=ft["z"],
                                out_t=yt)
    for _ in range(3):
        fused_token()
    torch.cuda.synchronize()
    he = HipEvents()
    fev = [he.pair() for _ in range(steps)]
    sev = [he.pair() for _ in range(steps)]
    for i in range(steps):
        ssm.ssm_set_kernel_timer("scan_step", *sev[i])
        he.record(fev[i][0], stream)
        fused_token()
        he.record(fev[i][1], stream)
    torch.cuda.synchronize()
    ssm.ssm_set_kernel_timer("scan_step", None, None)
    ftok = sum(he.elapsed_ms(*pr) for pr in fev) / steps
    fscan = sum(he.elapsed_ms(*pr) for pr in sev) / steps
    he.destroy()
    out["fused"] = {"token_ms": ftok, "tokens_per_s": Bd / (ftok * 1e-3),
                    "scan_step_kernel_ms": fscan}

    # the same token in one launch (ssm_decode_step)
    def one_launch():
        ssm.ssm_decode_step(hf, state, cx, c["W"], bias, ft["delta_raw"], f["A"], ft["Bm"],
                            ft["Cm"], f["Dv"], delta_bias=f["delta_bias"], delta_softplus=True,
                            z_t=ft["z"], out_t=yt)
    for _ in range(3):
        one_launch()
    torch.cuda.synchronize()
    he = HipEvents()
    oev = [he.pair() for _ in range(steps)]
    kev1 = [he.pair() for _ in range(steps)]
    for i in range(steps):
        ssm.ssm_set_kernel_timer("decode_step", *kev1[i])
        he.record(oev[i][0], stream)
        one_launch()
        he.record(oev[i][1], stream)
    torch.cuda.synchronize()
    ssm.ssm_set_kernel_timer("decode_step", None, None)
    otok = sum(he.elapsed_ms(*pr) for pr in oev) / steps
    okern = sum(he.elapsed_ms(*pr) for pr in kev1) / steps
    he.destroy()
    out["fused_one_launch"] = {"token_ms": otok, "tokens_per_s": Bd / (otok * 1e-3),
                               "kernel_ms": okern}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mamba-2.8b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-channels", type=int, default=0,
                    help="channels in the oracle's sample (default: about 10-30 s of CPU work)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the scan library runs on one GPU: every figure is one GPU's "
                          "throughput; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch

    from selective_state_space_02_amd import binding as ssm
    from selective_state_space_02_amd import synth
    from selective_state_space_02_amd.workloads import BY_NAME

    w = BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ssm.load()
    print(f"[bench] workload {w.name}: generating inputs", file=sys.stderr, flush=True)

    cpu_inputs = (synth.scan_inputs(w, args.seed), synth.conv_inputs(w, args.seed),
                  synth.rms_inputs(w, args.seed))
    p, c, r = ({k: v.to(dev) for k, v in d.items()} for d in cpu_inputs)
    # the statistic the RMSNorm forward saves for its backward (setup, untimed)
    _, r["rms"] = ssm.rmsnorm_fwd(r["x"], r["scale"], synth.RMS_EPS)
    f32 = torch.float32
    code = ssm.SSM_BF16 if w.dtype == "bf16" else ssm.SSM_F32
    B, L, D, N, K = w.B, w.L, w.D, w.N, w.K
    # every buffer allocated once, outside the timed region
    y = torch.empty_like(p["x"])
    ckpt = ssm.new_ckpt(B, L, D, N, dev)
    ws_f = torch.empty(max(1, ssm.ssm_scan_fwd_workspace_bytes(B, L, D, N, code)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, ssm.ssm_scan_bwd_workspace_bytes(B, L, D, N, code, True)), dtype=torch.uint8, device=dev)
    dx = torch.empty_like(p["x"])
    ddelta = torch.empty_like(p["x"])
    dA = torch.zeros((D, N), dtype=f32, device=dev)
    dB = torch.empty((B, L, N), dtype=f32, device=dev)
    dC = torch.empty((B, L, N), dtype=f32, device=dev)
    dD = torch.zeros((D,), dtype=f32, device=dev)
    cdx = torch.empty_like(c["x"])
    dW = torch.zeros((D, K), dtype=f32, device=dev)
    db = torch.zeros((D,), dtype=f32, device=dev)
    ws_c = torch.empty(max(1, ssm.conv1d_causal_bwd_workspace_bytes(B, L, D, K, code)), dtype=torch.uint8, device=dev)
    rdx = torch.empty_like(r["x"])
    dscale = torch.zeros((w.rms_dim,), dtype=f32, device=dev)
    ws_r = torch.empty(max(1, ssm.rmsnorm_bwd_workspace_bytes(w.rms_rows, w.rms_dim, code)), dtype=torch.uint8, device=dev)

    def call_fwd():
        ssm.ssm_scan_fwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], y=y, ckpt=ckpt, ws=ws_f)

    def call_bwd():
        ssm.ssm_scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["Dv"], p["dy"], ckpt=ckpt,
                         dx=dx, ddelta=ddelta, dA=dA, dB=dB, dC=dC, dD=dD, ws=ws_b)

    def call_conv():
        ssm.conv1d_causal_bwd(c["x"], c["W"], c["dout"], dx=cdx, dW=dW, db=db, ws=ws_c)

    def call_rms():
        ssm.rmsnorm_bwd(r["dy"], r["x"], r["scale"], r["rms"], dx=rdx, dscale=dscale, ws=ws_r)

    calls = [("scan_fwd", call_fwd), ("scan_bwd", call_bwd), ("conv_bwd", call_conv), ("rms_bwd", call_rms)]
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()

    # events: per call (on torch's current stream, the stream every call is launched on)
    # and around the backward main kernel through the library's timing hook
    K_ = args.steps
    he = HipEvents()
    ev = {name: [he.pair() for _ in range(K_)] for name, _ in calls}
    kernels = ["bwd_main", "fwd_output", "fwd_summary", "bwd_summary", "conv_bwd", "rms_bwd"]
    kev = {k: [he.pair() for _ in range(K_)] for k in kernels}
    stream = torch.cuda.current_stream(dev).cuda_stream
    print(f"[bench] timing {K_} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K_):
        for k in kernels:
            ssm.ssm_set_kernel_timer(k, *kev[k][i])
        for name, f in calls:
            he.record(ev[name][i][0], stream)
            f()
            he.record(ev[name][i][1], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in kernels:
        ssm.ssm_set_kernel_timer(k, None, None)

    ms_per_step = (t1 - t0) * 1e3 / K_
    call_ms = {name: sum(he.elapsed_ms(*pr) for pr in ev[name]) / K_ for name, _ in calls}

    def kernel_ms(k):
        vals = [he.elapsed_ms(*pr) for pr in kev[k]]
        if any(v is None for v in vals):
            return None        # a kernel this workload does not launch
        return sum(vals) / K_
    kern_ms = {k: kernel_ms(k) for k in kernels}
    he.destroy()

    tokch = B * L * D
    ab = algorithmic_bytes(w)
    step_bytes = sum(ab.values())
    scan_call_ms = call_ms["scan_fwd"] + call_ms["scan_bwd"]  # instrumented loop
    print(f"[bench] timing {K_} scan forward+backward pairs back to back", file=sys.stderr,
          flush=True)
    scan_ms = measure_scan_back_to_back(call_fwd, call_bwd, K_)
    value = tokch / (scan_ms * 1e-3)  # the metric: scan forward + backward
    main_ms = kern_ms["bwd_main"]
    main_gbps = bwd_main_bytes(w) / (main_ms * 1e-3) / 1e9
    updates = B * L * D * N
    main_ops = (BWD_MAIN_VALU_PER_UPDATE + BWD_MAIN_EXP_PER_UPDATE) * updates
    slots = counter_valu_slots(w.name)
    valu_floor_ms = slots / VALU_WAVE_INSTR_PER_S * 1e3 if slots else None

    layer_fwd = measure_layer_forward(w, c, r, args.seed, K_, dev)
    decode = measure_decode(w, args.seed, K_, dev)
    conv_silu = measure_conv_silu(w, c, args.seed, K_, dev)
    scan_fused = measure_scan_fused(w, args.seed, K_, dev)
    scan_fused["overhead_vs_plain_ms"] = (scan_fused["call_ms"]["fused_fwd"] +
                                          scan_fused["call_ms"]["fused_bwd"] - scan_call_ms)

    ckpt_iv = measure_ckpt_intervals(w, p, K_, dev)
    alpha = measure_alpha_scan(args.seed, K_, dev)
    graph_step = measure_graph_step(calls, K_, dev)
    copy_gbps = measure_copy_GBps(dev)

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=f32, device=dev)
        b2 = torch.empty_like(a)
        b2.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens*channels/s",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "L": L, "D": D, "N": N, "K": K,
                   "io_dtype": w.dtype, "rms_rows": w.rms_rows, "rms_dim": w.rms_dim,
                   "step": "ssm_scan_fwd + ssm_scan_bwd + conv1d_causal_bwd + rmsnorm_bwd"},
        "scan_fwd_bwd_ms": scan_ms,
        "scan_fwd_bwd_instrumented_ms": scan_call_ms,
        "step_tokens_channels_per_s": tokch / (ms_per_step * 1e-3),
        "hbm": {"algorithmic_bytes_per_step": step_bytes,
                "GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
                "frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                "scan_fwd_bwd_GBps": (ab["scan_fwd"] + ab["scan_bwd"]) / (scan_ms * 1e-3) / 1e9,
                "conv_bwd_GBps": ab["conv_bwd"] / (call_ms["conv_bwd"] * 1e-3) / 1e9,
                "rms_bwd_GBps": ab["rms_bwd"] / (call_ms["rms_bwd"] * 1e-3) / 1e9,
                "copy_GBps": copy_gbps,
                "frac_of_copy": step_bytes / (ms_per_step * 1e-3) / 1e9 / copy_gbps},
        "call_ms": call_ms,
        "kernel_ms": kern_ms,
        "roofline": {
            "kernel": "k_bwd_main (scan backward main)",
            "bound": "hbm",
            "achieved": main_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": main_gbps / HBM_PEAK_GBPS,
            "traffic": counter_traffic(w.name),
            "avg_launch_ms": main_ms,
            "algorithmic_bytes_per_launch": bwd_main_bytes(w),
            # `bound` names the roof `frac` is taken against (the metric's: HBM); the
            # resource that limits the kernel is its VALU issue rate
            "limited_by": "valu_issue",
            # what actually binds the kernel: VALU issue.  Its issue time from the
            # committed counter record (null once the kernel's sources changed since),
            # and the method's own op count against the non-packed lane-op peak
            "valu": {
                "issue_slots_per_launch": slots,
                "issue_floor_ms": valu_floor_ms,
                "frac_of_issue_roof": valu_floor_ms / main_ms if valu_floor_ms else None,
                "algorithmic_ops_per_update": BWD_MAIN_VALU_PER_UPDATE + BWD_MAIN_EXP_PER_UPDATE,
                "algorithmic_lane_ops_per_s": main_ops / (main_ms * 1e-3),
                "lane_ops_peak_per_s": LANE_OPS_PEAK,
                "frac_of_lane_op_peak": main_ops / (main_ms * 1e-3) / LANE_OPS_PEAK,
                "fp32_nonpacked_peak_tflops": FP32_NONPACKED_PEAK_TFLOPS,
            },
        },
    }
    out["layer_forward"] = layer_fwd
    out["conv_silu"] = conv_silu
    out["scan_fused"] = scan_fused
    out["decode"] = decode
    out["ckpt_interval"] = ckpt_iv
    out["alpha_scan"] = alpha
    out["graph_step"] = graph_step
    if not args.no_cpu_baseline:
        sample = args.cpu_sample_channels or max(16, min(w.D, 2048))
        print(f"[bench] cpu baseline: oracle on {sample} channels", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, cpu_inputs, sample, "timed on this host's cores")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
