"""C-ABI boundary tests that need no GPU.

The library must load, export every function ``include/ssm_scan.h`` declares, and reject
bad arguments on the host before any HIP call: null required pointers, non-positive or
overflowing sizes, unsupported N / K / dtype / M, misaligned pointers and too-small
workspaces each return their documented code with a message.  Fake (never dereferenced)
device addresses are passed; every call here is rejected by validation, so no kernel is
launched and no device memory is touched.
"""
import ctypes
import os
import re

import pytest

from selective_state_space_02_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm_scan.h")

FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
MIS = FAKE + 4                 # misaligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+)\s*\(", src)
    skip = {"if", "for", "while", "sizeof", "return"}
    return sorted({n for n in names if n not in skip})


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("ssm_scan_fwd", "ssm_scan_bwd", "conv1d_causal_bwd", "rmsnorm_bwd",
              "conv1d_causal_fwd", "rmsnorm_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = b.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"symbol {name} declared in ssm_scan.h is not exported"
    assert set(b.EXPORTS) == set(declared_functions())


def test_version_and_empty_error():
    assert b.version().startswith("ssmscan-gfx950")


def _fwd(lib, B=2, L=64, D=32, N=16, dtype=0, x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE,
         Dv=FAKE, h0=None, y=FAKE, ckpt=None, h_last=None, ws=None, ws_bytes=0):
    return lib.ssm_scan_fwd(None, dtype, B, L, D, N, x, delta, A, Bm, Cm, Dv, h0, y, ckpt,
                            h_last, ws, ws_bytes)


def _bwd(lib, B=2, L=64, D=32, N=16, dtype=0, ckpt=FAKE, ws=None, ws_bytes=0, **kw):
    p = dict(x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dv=FAKE, h0=None, dy=FAKE,
             dx=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=FAKE, dh0=None)
    p.update(kw)
    return lib.ssm_scan_bwd(None, dtype, B, L, D, N, p["x"], p["delta"], p["A"], p["Bm"],
                            p["Cm"], p["Dv"], p["h0"], p["dy"], ckpt, p["dx"], p["ddelta"],
                            p["dA"], p["dB"], p["dC"], p["dD"], p["dh0"], ws, ws_bytes)


def _ffwd(lib, B=2, L=64, D=32, N=16, dtype=0, ws=None, ws_bytes=0, **kw):
    p = dict(x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dv=FAKE, h0=None, delta_bias=None,
             delta_softplus=1, z=None, out=FAKE, y_save=None, ckpt=None, h_last=None)
    p.update(kw)
    return lib.ssm_scan_fused_fwd(None, dtype, B, L, D, N, p["x"], p["delta"], p["A"], p["Bm"],
                                  p["Cm"], p["Dv"], p["h0"], p["delta_bias"],
                                  p["delta_softplus"], p["z"], p["out"], p["y_save"], p["ckpt"],
                                  p["h_last"], ws, ws_bytes)


def _fbwd(lib, B=2, L=64, D=32, N=16, dtype=0, ckpt=FAKE, ws=None, ws_bytes=0, **kw):
    p = dict(x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dv=FAKE, h0=None, delta_bias=None,
             delta_softplus=1, z=None, y_save=None, dout=FAKE, dx=FAKE, ddelta=FAKE, dA=FAKE,
             dB=FAKE, dC=FAKE, dD=FAKE, dh0=None, dz=None, ddelta_bias=None)
    p.update(kw)
    return lib.ssm_scan_fused_bwd(None, dtype, B, L, D, N, p["x"], p["delta"], p["A"], p["Bm"],
                                  p["Cm"], p["Dv"], p["h0"], p["delta_bias"],
                                  p["delta_softplus"], p["z"], p["y_save"], p["dout"], ckpt,
                                  p["dx"], p["ddelta"], p["dA"], p["dB"], p["dC"], p["dD"],
                                  p["dh0"], p["dz"], p["ddelta_bias"], ws, ws_bytes)


def test_scan_fused_validation():
    lib = b.load()
    # sizes and dtypes as the plain scan
    assert _ffwd(lib, N=3) == b.SSM_ERR_UNSUPPORTED
    assert _fbwd(lib, L=0) == b.SSM_ERR_ARG
    assert _ffwd(lib, dtype=4) == b.SSM_ERR_UNSUPPORTED
    for name in ("x", "delta", "A", "Bm", "Cm", "Dv", "out"):
        assert _ffwd(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
    for name in ("dout", "dx", "ddelta", "dA", "dB", "dC", "dD"):
        assert _fbwd(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
    # optional pointers are checked for alignment when given
    for name in ("delta_bias", "z", "y_save", "h_last"):
        assert _ffwd(lib, **{name: MIS}) == b.SSM_ERR_ALIGN, name
    for name in ("delta_bias", "z", "y_save", "dz", "ddelta_bias", "dh0"):
        assert _fbwd(lib, **{name: MIS}) == b.SSM_ERR_ALIGN, name
    # the softplus switch is 0 or 1
    assert _ffwd(lib, delta_softplus=2) == b.SSM_ERR_ARG
    assert "delta_softplus" in b.last_error()
    assert _fbwd(lib, delta_softplus=-1) == b.SSM_ERR_ARG
    # the gate's pointers come together
    assert _ffwd(lib, y_save=FAKE) == b.SSM_ERR_ARG
    assert "y_save" in b.last_error()
    assert _fbwd(lib, z=FAKE) == b.SSM_ERR_ARG
    assert _fbwd(lib, z=FAKE, y_save=FAKE) == b.SSM_ERR_ARG
    assert _fbwd(lib, z=FAKE, dz=FAKE) == b.SSM_ERR_ARG
    assert _fbwd(lib, dz=FAKE) == b.SSM_ERR_ARG
    assert _fbwd(lib, y_save=FAKE) == b.SSM_ERR_ARG
    # workspaces as the plain scan's
    need = b.ssm_scan_bwd_workspace_bytes(2, 64, 32, 16, 0, 1)
    assert _fbwd(lib, ws=FAKE, ws_bytes=need - 1) == b.SSM_ERR_WORKSPACE


@pytest.mark.parametrize("dims", [(0, 8, 8, 16), (2, 0, 8, 16), (2, 8, 0, 16), (2, 8, 8, 0),
                                  (-1, 8, 8, 16)])
def test_scan_rejects_nonpositive_sizes(dims):
    lib = b.load()
    B, L, D, N = dims
    assert _fwd(lib, B, L, D, N) == b.SSM_ERR_ARG
    assert "positive" in b.last_error()
    assert _bwd(lib, B, L, D, N) == b.SSM_ERR_ARG


@pytest.mark.parametrize("N", [1, 2, 3, 5, 12, 32, 64])
def test_scan_rejects_unsupported_state_size(N):
    lib = b.load()
    assert _fwd(lib, N=N) == b.SSM_ERR_UNSUPPORTED
    assert "state size" in b.last_error()
    assert _bwd(lib, N=N) == b.SSM_ERR_UNSUPPORTED


def test_scan_rejects_unsupported_dtype_and_grid():
    lib = b.load()
    assert _fwd(lib, dtype=2) == b.SSM_ERR_UNSUPPORTED
    # the batch is not capped by a grid dimension of 65535 any more (the grid is 1-D); only
    # (batch rows) x (64-channel groups) beyond one launch's 2^31 - 1 workgroups is refused
    assert _fwd(lib, B=1 << 31, L=1, D=64) == b.SSM_ERR_UNSUPPORTED
    assert "grid" in b.last_error()
    assert _bwd(lib, B=1 << 31, L=1, D=64) == b.SSM_ERR_UNSUPPORTED


def test_scan_rejects_overflowing_sizes():
    lib = b.load()
    assert _fwd(lib, B=60000, L=1 << 30, D=1 << 20) == b.SSM_ERR_ARG
    assert "overflow" in b.last_error()


@pytest.mark.parametrize("missing", ["x", "delta", "A", "Bm", "Cm", "Dv", "y"])
def test_fwd_rejects_null_required_pointer(missing):
    lib = b.load()
    assert _fwd(lib, **{missing: None}) == b.SSM_ERR_ARG
    assert missing in b.last_error()


@pytest.mark.parametrize("missing", ["x", "delta", "A", "Bm", "Cm", "Dv", "dy", "dx", "ddelta",
                                     "dA", "dB", "dC", "dD"])
def test_bwd_rejects_null_required_pointer(missing):
    lib = b.load()
    assert _bwd(lib, **{missing: None}) == b.SSM_ERR_ARG
    assert missing in b.last_error()


@pytest.mark.parametrize("bad", ["x", "Bm", "y", "h0", "ckpt", "h_last"])
def test_fwd_rejects_misaligned_pointer(bad):
    lib = b.load()
    assert _fwd(lib, **{bad: MIS}) == b.SSM_ERR_ALIGN
    assert bad in b.last_error()


def test_bwd_rejects_misaligned_pointer():
    lib = b.load()
    assert _bwd(lib, dh0=MIS) == b.SSM_ERR_ALIGN
    assert _bwd(lib, dB=MIS) == b.SSM_ERR_ALIGN
    assert _bwd(lib, ckpt=MIS) == b.SSM_ERR_ALIGN


def test_scan_rejects_small_workspace():
    lib = b.load()
    # a workload with several coarse chunks needs a forward workspace
    B, L, D, N = 2, 4096, 64, 16
    need = b.ssm_scan_fwd_workspace_bytes(B, L, D, N, 0)
    assert need > 0
    assert _fwd(lib, B, L, D, N, ws=FAKE, ws_bytes=need - 1) == b.SSM_ERR_WORKSPACE
    assert "workspace" in b.last_error()
    assert _fwd(lib, B, L, D, N, ws=None, ws_bytes=need) == b.SSM_ERR_WORKSPACE
    assert _fwd(lib, B, L, D, N, ws=MIS, ws_bytes=need) == b.SSM_ERR_ALIGN
    needb = b.ssm_scan_bwd_workspace_bytes(B, L, D, N, 0, 1)
    assert _bwd(lib, B, L, D, N, ws=FAKE, ws_bytes=needb - 1) == b.SSM_ERR_WORKSPACE


def test_workspace_queries_are_consistent():
    for (B, L, D, N) in [(1, 1, 1, 4), (2, 8, 8, 4), (256, 32, 64, 16), (8, 2048, 1536, 16),
                         (2, 16384, 5120, 16), (3, 333, 80, 8)]:
        interval = 8 if N == 16 else 16   # the state before every interval-th step
        assert b.ssm_scan_ckpt_bytes(B, L, D, N) == B * (-(-L // interval)) * D * N * 4
        with_ck = b.ssm_scan_bwd_workspace_bytes(B, L, D, N, 1, 1)
        without = b.ssm_scan_bwd_workspace_bytes(B, L, D, N, 1, 0)
        # recomputing the forward needs room for the checkpoints
        assert without >= with_ck + b.ssm_scan_ckpt_bytes(B, L, D, N)
        assert with_ck >= 2 * B * L * N * 4      # the dB and dC partials
    assert b.ssm_scan_ckpt_bytes(0, 1, 1, 4) == 0
    assert b.ssm_scan_fwd_workspace_bytes(1, 1, 1, 4, 0) == 0


def _conv(lib, B=2, L=64, D=32, K=4, dtype=0, x=FAKE, W=FAKE, bias=None, act=0, dout=FAKE,
          dx=FAKE, dW=FAKE, db=FAKE, ws=None, ws_bytes=0):
    return lib.conv1d_causal_bwd(None, dtype, B, L, D, K, x, W, bias, act, dout, dx, dW, db,
                                 ws, ws_bytes)


def test_conv_validation():
    lib = b.load()
    assert _conv(lib, K=0) == b.SSM_ERR_ARG
    assert _conv(lib, K=9) == b.SSM_ERR_UNSUPPORTED
    assert _conv(lib, L=0) == b.SSM_ERR_ARG
    assert _conv(lib, dtype=5) == b.SSM_ERR_UNSUPPORTED
    assert _conv(lib, act=2) == b.SSM_ERR_UNSUPPORTED
    assert "activation" in b.last_error()
    assert _conv(lib, act=-1) == b.SSM_ERR_UNSUPPORTED
    assert _conv(lib, act=1, bias=MIS) == b.SSM_ERR_ALIGN    # optional, but aligned if given
    for name in ("x", "W", "dout", "dx", "dW", "db"):
        assert _conv(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
        assert _conv(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    need = b.conv1d_causal_bwd_workspace_bytes(2, 64, 32, 4, 0)
    assert need > 0
    assert _conv(lib, ws=FAKE, ws_bytes=need - 1) == b.SSM_ERR_WORKSPACE
    # no 32-bit size limit on D (per-row descriptors); only a grid of more than 2^31 - 1
    # workgroups (batch rows x channel groups) is refused
    assert _conv(lib, B=1 << 31, L=1, D=64) == b.SSM_ERR_UNSUPPORTED
    assert "grid" in b.last_error()
    assert b.conv1d_causal_bwd_workspace_bytes(1, 2, 1 << 27, 4, 1) > 0


def _rms(lib, R=64, M=128, dtype=0, dy=FAKE, x=FAKE, scale=FAKE, rms=FAKE, dx=FAKE,
         dscale=FAKE, ws=None, ws_bytes=0):
    return lib.rmsnorm_bwd(None, dtype, R, M, dy, x, scale, rms, dx, dscale, ws, ws_bytes)


def test_rms_validation():
    lib = b.load()
    assert _rms(lib, R=0) == b.SSM_ERR_ARG
    assert _rms(lib, M=-3) == b.SSM_ERR_ARG
    assert _rms(lib, dtype=7) == b.SSM_ERR_UNSUPPORTED
    # rows of any length are supported (the looped path beyond 16 column groups per
    # lane); only a row whose column slabs would exceed one launch's grid is refused
    assert _rms(lib, R=1, M=(1 << 40) + 1, dtype=0) == b.SSM_ERR_UNSUPPORTED
    assert "grid" in b.last_error()
    for name in ("dy", "x", "scale", "rms", "dx", "dscale"):
        assert _rms(lib, **{name: None}) == b.SSM_ERR_ARG
        assert _rms(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    need = b.rmsnorm_bwd_workspace_bytes(64, 128, 0)
    assert need > 0
    assert _rms(lib, ws=FAKE, ws_bytes=need - 1) == b.SSM_ERR_WORKSPACE
    assert b.rmsnorm_bwd_workspace_bytes(10, 8192, 1) > 0
    # the looped path (odd M, or M past 16 column groups per lane) also holds the per-row
    # coefficients: R floats more than the block partials
    for R, M, dt in ((10, 8193, 1), (10, 1500, 0), (10, 12288, 1), (10, 8192 * 4, 0)):
        assert b.rmsnorm_bwd_workspace_bytes(R, M, dt) > 0


def _conv_fwd(lib, B=2, L=64, D=32, K=4, dtype=0, x=FAKE, W=FAKE, bias=None, act=0, out=FAKE):
    return lib.conv1d_causal_fwd(None, dtype, B, L, D, K, x, W, bias, act, out)


def test_conv_fwd_validation():
    lib = b.load()
    assert _conv_fwd(lib, K=0) == b.SSM_ERR_ARG
    assert _conv_fwd(lib, K=9) == b.SSM_ERR_UNSUPPORTED
    assert _conv_fwd(lib, B=0) == b.SSM_ERR_ARG
    assert _conv_fwd(lib, dtype=2) == b.SSM_ERR_UNSUPPORTED
    assert _conv_fwd(lib, act=3) == b.SSM_ERR_UNSUPPORTED
    for name in ("x", "W", "out"):
        assert _conv_fwd(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
        assert _conv_fwd(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    assert _conv_fwd(lib, bias=MIS) == b.SSM_ERR_ALIGN     # optional, but aligned if given
    assert _conv_fwd(lib, B=1 << 31, L=1, D=64) == b.SSM_ERR_UNSUPPORTED
    assert "grid" in b.last_error()


def _rms_fwd(lib, R=64, M=128, dtype=0, x=FAKE, residual=None, scale=FAKE, eps=1e-5, y=FAKE,
             rms=FAKE, residual_out=None):
    return lib.rmsnorm_fwd(None, dtype, R, M, x, residual, scale, eps, y, rms, residual_out)


def test_rms_fwd_validation():
    lib = b.load()
    assert _rms_fwd(lib, R=0) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, M=0) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, eps=-1.0) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, eps=float("nan")) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, eps=float("inf")) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, dtype=3) == b.SSM_ERR_UNSUPPORTED
    for name in ("x", "scale", "y", "rms"):
        assert _rms_fwd(lib, **{name: None}) == b.SSM_ERR_ARG
        assert _rms_fwd(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    # the residual stream: both pointers or neither, aligned
    assert _rms_fwd(lib, residual=FAKE) == b.SSM_ERR_ARG
    assert "residual" in b.last_error()
    assert _rms_fwd(lib, residual_out=FAKE) == b.SSM_ERR_ARG
    assert _rms_fwd(lib, residual=MIS, residual_out=FAKE) == b.SSM_ERR_ALIGN
    assert _rms_fwd(lib, residual=FAKE, residual_out=MIS) == b.SSM_ERR_ALIGN


def _step(lib, B=2, D=32, N=16, dtype=0, **kw):
    p = dict(h=FAKE, x_t=FAKE, delta_t=FAKE, A=FAKE, B_t=FAKE, C_t=FAKE, Dv=FAKE, y_t=FAKE)
    p.update(kw)
    return lib.ssm_scan_step(None, dtype, B, D, N, p["h"], p["x_t"], p["delta_t"], p["A"],
                             p["B_t"], p["C_t"], p["Dv"], p["y_t"])


def test_scan_step_validation():
    lib = b.load()
    assert _step(lib, N=3) == b.SSM_ERR_UNSUPPORTED
    assert _step(lib, B=0) == b.SSM_ERR_ARG
    assert _step(lib, D=-1) == b.SSM_ERR_ARG
    assert _step(lib, B=1 << 31, D=64) == b.SSM_ERR_UNSUPPORTED  # beyond one launch's grid
    assert _step(lib, dtype=9) == b.SSM_ERR_UNSUPPORTED
    for name in ("h", "x_t", "delta_t", "A", "B_t", "C_t", "Dv", "y_t"):
        assert _step(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
        assert _step(lib, **{name: MIS}) == b.SSM_ERR_ALIGN


def _cstep(lib, B=2, D=32, K=4, dtype=0, state=FAKE, x_t=FAKE, W=FAKE, bias=None, act=0,
           out_t=FAKE):
    return lib.conv1d_causal_step(None, dtype, B, D, K, state, x_t, W, bias, act, out_t)


def _fstep(lib, B=2, D=32, N=16, dtype=0, **kw):
    p = dict(h=FAKE, x_t=FAKE, delta_t=FAKE, A=FAKE, B_t=FAKE, C_t=FAKE, Dv=FAKE,
             delta_bias=None, delta_softplus=1, z_t=None, out_t=FAKE)
    p.update(kw)
    return lib.ssm_scan_fused_step(None, dtype, B, D, N, p["h"], p["x_t"], p["delta_t"], p["A"],
                                   p["B_t"], p["C_t"], p["Dv"], p["delta_bias"],
                                   p["delta_softplus"], p["z_t"], p["out_t"])


def _dstep(lib, B=2, D=32, N=16, K=4, dtype=0, **kw):
    p = dict(h=FAKE, conv_state=FAKE, x_t=FAKE, W=FAKE, conv_bias=None, delta_t=FAKE, A=FAKE,
             B_t=FAKE, C_t=FAKE, Dv=FAKE, delta_bias=None, delta_softplus=1, z_t=None,
             out_t=FAKE)
    p.update(kw)
    return lib.ssm_decode_step(None, dtype, B, D, N, K, p["h"], p["conv_state"], p["x_t"], p["W"],
                               p["conv_bias"], p["delta_t"], p["A"], p["B_t"], p["C_t"], p["Dv"],
                               p["delta_bias"], p["delta_softplus"], p["z_t"], p["out_t"])


def test_decode_step_validation():
    lib = b.load()
    assert _dstep(lib, N=5) == b.SSM_ERR_UNSUPPORTED
    assert _dstep(lib, K=0) == b.SSM_ERR_ARG
    assert _dstep(lib, K=9) == b.SSM_ERR_UNSUPPORTED
    assert _dstep(lib, B=0) == b.SSM_ERR_ARG
    assert _dstep(lib, delta_softplus=3) == b.SSM_ERR_ARG
    for name in ("h", "conv_state", "x_t", "W", "delta_t", "A", "B_t", "C_t", "Dv", "out_t"):
        assert _dstep(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
    for name in ("conv_bias", "delta_bias", "z_t", "h"):
        assert _dstep(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    # a width-1 conv has no window: conv_state may be NULL
    assert _dstep(lib, K=1, conv_state=MIS) == b.SSM_ERR_ALIGN


def test_scan_fused_step_validation():
    lib = b.load()
    assert _fstep(lib, N=5) == b.SSM_ERR_UNSUPPORTED
    assert _fstep(lib, B=0) == b.SSM_ERR_ARG
    assert _fstep(lib, delta_softplus=2) == b.SSM_ERR_ARG
    for name in ("h", "x_t", "delta_t", "A", "B_t", "C_t", "Dv", "out_t"):
        assert _fstep(lib, **{name: None}) == b.SSM_ERR_ARG
        assert name in b.last_error()
    for name in ("delta_bias", "z_t"):
        assert _fstep(lib, **{name: MIS}) == b.SSM_ERR_ALIGN


def test_conv_step_validation():
    lib = b.load()
    assert _cstep(lib, K=0) == b.SSM_ERR_ARG
    assert _cstep(lib, K=9) == b.SSM_ERR_UNSUPPORTED
    assert _cstep(lib, D=0) == b.SSM_ERR_ARG
    assert _cstep(lib, dtype=4) == b.SSM_ERR_UNSUPPORTED
    assert _cstep(lib, act=5) == b.SSM_ERR_UNSUPPORTED
    assert _cstep(lib, B=1 << 20, D=1 << 19) == b.SSM_ERR_ARG   # beyond one thread per (b, d)
    for name in ("state", "x_t", "W", "out_t"):
        assert _cstep(lib, **{name: None}) == b.SSM_ERR_ARG
        assert _cstep(lib, **{name: MIS}) == b.SSM_ERR_ALIGN
    assert _cstep(lib, bias=MIS) == b.SSM_ERR_ALIGN
    # a width-1 conv has no window: state may be NULL (still checked for alignment if given)
    assert _cstep(lib, K=1, state=MIS) == b.SSM_ERR_ALIGN


def test_error_message_is_per_call():
    lib = b.load()
    assert _fwd(lib, N=3) == b.SSM_ERR_UNSUPPORTED
    msg1 = b.last_error()
    assert _conv(lib, K=9) == b.SSM_ERR_UNSUPPORTED
    assert b.last_error() != msg1


def test_binding_rejects_cpu_and_strided_tensors():
    import torch
    x = torch.zeros(2, 8, 8)
    with pytest.raises(ValueError, match="GPU"):
        b._ptr(x, "x")
    # strided views never reach the library
    class FakeCuda:
        pass
    with pytest.raises(TypeError):
        b._ptr(FakeCuda(), "x")
    # activations are named; an unknown one is rejected before any pointer is formed
    assert b._act_code("none") == 0 and b._act_code("silu") == 1
    with pytest.raises(ValueError, match="activation"):
        b._act_code("gelu")


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", "/nonexistent/libssmscan.so")
    with pytest.raises(RuntimeError, match="not built"):
        b.load()


def test_no_oracle_in_product_sources():
    # the product (library sources and binding) never references the oracle
    pkg = os.path.join(ROOT, "selective_state_space_02_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
                assert "liboracle" not in src, f
    csrc = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert "ssm_scan.h" not in csrc and "common.hpp" not in csrc


def _fwd_every(lib, every, B=2, L=64, D=32, N=16, ckpt=FAKE, **kw):
    p = dict(x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dv=FAKE, h0=None, y=FAKE, h_last=None)
    p.update(kw)
    return lib.ssm_scan_fwd_every(None, 0, B, L, D, N, p["x"], p["delta"], p["A"], p["Bm"],
                                  p["Cm"], p["Dv"], p["h0"], p["y"], ckpt, p["h_last"], every,
                                  None, 0)


def _bwd_every(lib, every, slabs, B=2, L=64, D=32, N=16, ckpt=FAKE, ws=None, ws_bytes=0, **kw):
    p = dict(x=FAKE, delta=FAKE, A=FAKE, Bm=FAKE, Cm=FAKE, Dv=FAKE, h0=None, dy=FAKE,
             dx=FAKE, ddelta=FAKE, dA=FAKE, dB=FAKE, dC=FAKE, dD=FAKE, dh0=None, dh_last=None)
    p.update(kw)
    return lib.ssm_scan_bwd_every(None, 0, B, L, D, N, p["x"], p["delta"], p["A"], p["Bm"],
                                  p["Cm"], p["Dv"], p["h0"], p["dy"], ckpt, p["dx"],
                                  p["ddelta"], p["dA"], p["dB"], p["dC"], p["dD"], p["dh0"],
                                  p["dh_last"], every, slabs, ws, ws_bytes)


@pytest.mark.parametrize("every,N", [(-16, 16), (24, 16), (8, 4), (8, 8), (4, 16), (17, 16)])
def test_checkpoint_interval_validation(every, N):
    # the interval is 0 (default), the default itself, or a positive multiple of 16 steps
    lib = b.load()
    assert _fwd_every(lib, every, N=N) == b.SSM_ERR_ARG
    assert "checkpoint interval" in b.last_error()
    assert _bwd_every(lib, every, 1, N=N) == b.SSM_ERR_ARG
    assert b.ssm_scan_ckpt_bytes_every(2, 64, 32, N, every) == 0
    assert b.ssm_scan_bwd_workspace_bytes_every(2, 64, 32, N, 0, 1, every, 1) == 0


def test_checkpoint_interval_slabs_and_sizes():
    lib = b.load()
    assert _bwd_every(lib, 64, 0) == b.SSM_ERR_ARG
    assert "slabs" in b.last_error()
    assert _bwd_every(lib, 64, 65537) == b.SSM_ERR_ARG
    assert b.ssm_scan_bwd_workspace_bytes_every(2, 64, 32, 16, 0, 1, 64, 65537) == 0
    assert b.ssm_scan_bwd_workspace_bytes_every(2, 64, 32, 16, 0, 1, 64, 65536) > 0
    assert b.ssm_scan_bwd_workspace_bytes_every(2, 64, 32, 16, 0, 1, 64, 0) == 0
    # the default interval through the new entry points is the plain call's plan
    assert b.ssm_scan_ckpt_bytes_every(2, 1000, 32, 16, 0) == b.ssm_scan_ckpt_bytes(2, 1000, 32, 16)
    assert b.ssm_scan_ckpt_bytes_every(2, 1000, 32, 16, 8) == b.ssm_scan_ckpt_bytes(2, 1000, 32, 16)
    assert b.ssm_scan_bwd_workspace_bytes_every(2, 1000, 32, 16, 0, 1, 0, 1) == \
        b.ssm_scan_bwd_workspace_bytes(2, 1000, 32, 16, 0, 1)
    # checkpoints shrink with the interval; the backward's workspace holds one slab's
    # regenerated states, so more slabs take less of it
    B, L, D, N = 2, 16384, 5120, 16
    dense = b.ssm_scan_ckpt_bytes(B, L, D, N)
    for every in (16, 64, 512):
        assert b.ssm_scan_ckpt_bytes_every(B, L, D, N, every) * (every // 8) == dense
    w1 = b.ssm_scan_bwd_workspace_bytes_every(B, L, D, N, 1, 1, 64, 1)
    w8 = b.ssm_scan_bwd_workspace_bytes_every(B, L, D, N, 1, 1, 64, 8)
    assert w8 < w1
    # a too-small workspace is refused before any launch
    assert _bwd_every(lib, 64, 8, B=B, L=L, D=D, N=N, ws=FAKE, ws_bytes=w8 - 1) == \
        b.SSM_ERR_WORKSPACE
    # the final state's gradient is optional, but aligned if given
    assert _bwd_every(lib, 0, 1, dh_last=MIS) == b.SSM_ERR_ALIGN
    assert "dh_last" in b.last_error()


def test_alpha_scan_validation():
    lib = b.load()

    def fwd(Bn=4, K=8, S=4, H=8, **kw):
        p = dict(a=FAKE, b=FAKE, Wc=FAKE, h0=None, h=FAKE)
        p.update(kw)
        return lib.ssm_alpha_scan_fwd(None, Bn, K, S, H, p["a"], p["b"], p["Wc"], p["h0"], p["h"])

    def bwd(Bn=4, K=8, S=4, H=8, ws=None, ws_bytes=0, **kw):
        p = dict(a=FAKE, b=FAKE, Wc=FAKE, dh=FAKE, da=FAKE, db=FAKE, dWc=FAKE, dh0=None)
        p.update(kw)
        return lib.ssm_alpha_scan_bwd(None, Bn, K, S, H, p["a"], p["b"], p["Wc"], p["dh"],
                                      p["da"], p["db"], p["dWc"], p["dh0"], ws, ws_bytes)
    for dims in ((0, 8, 4, 8), (4, 0, 4, 8), (4, 8, 0, 8), (4, 8, 4, -1)):
        assert fwd(*dims) == b.SSM_ERR_ARG
        assert bwd(*dims) == b.SSM_ERR_ARG
    assert fwd(S=1025) == b.SSM_ERR_UNSUPPORTED and "state size" in b.last_error()
    assert bwd(S=1025) == b.SSM_ERR_UNSUPPORTED
    for name in ("a", "b", "Wc", "h"):
        assert fwd(**{name: None}) == b.SSM_ERR_ARG and name in b.last_error()
        assert fwd(**{name: MIS}) == b.SSM_ERR_ALIGN
    assert fwd(h0=MIS) == b.SSM_ERR_ALIGN
    for name in ("a", "b", "Wc", "dh", "da", "db", "dWc"):
        assert bwd(**{name: None}) == b.SSM_ERR_ARG and name in b.last_error()
    need = b.load().ssm_alpha_scan_bwd_workspace_bytes(4, 8, 4, 8)
    assert need >= 4 * 8 * 4 * 4 + 4 * 4 * 4
    assert bwd(ws=FAKE, ws_bytes=need - 1) == b.SSM_ERR_WORKSPACE


def test_chunk_plan_prefers_long_chunks_while_the_grid_stays_full():
    # (forward, backward) coarse chunks.  The 2 x 16384 x 5120 layer keeps its
    # grid-target plan; where that plan would cut chunks of 2-4 tiles, chunks grow
    # towards 16 tiles (256 steps) as long as 1024 workgroups remain; narrow problems
    # keep short chunks to fill the GPU; one tile is one chunk.
    assert b.scan_chunks(2, 16384, 5120, 16) == (54, 32)
    assert b.scan_chunks(8, 2048, 1536, 16) == (8, 8)
    assert b.scan_chunks(4, 1000, 4100, 16) == (5, 5)
    assert b.scan_chunks(1, 16384, 64, 16) == (512, 512)
    assert b.scan_chunks(2, 8, 8, 4) == (1, 1)
